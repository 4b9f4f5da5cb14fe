// Sparse layers with KV Reuse, specialised for bf16 and head dim 128: one
// kernel for many queries (prefill-shaped calls) and, further down, one for
// few index lists (decode-shaped calls). Same contract as sparse_attn.hip:
// every sparse layer attends, with one softmax, over the same index set and
// the same K/V as the full layer (HySparse2 pages: "Xiaomi Unveils HySparse2
// for Faster Long-Context AI", sections "Two-Level KV Sharing" and
// "Token-Level Selection and Unified Local Access").
//
// The pass is bound by the gather from HBM, so the design keeps many gathers
// in flight without spending registers on them: one work-group serves one
// (sequence, query, KV head); its waves gather 32-key tiles of the selected
// K and V rows straight into a two-stage LDS ring (global_load_lds, the
// next tile in flight while one is used), and each wave then computes one
// 16-row block of (layer, head-of-group) rows from LDS. Every selected row
// is read from HBM once for all heads and layers of the group. The ring is
// kept shallow so that four work-groups fit a CU (36.6 KB of LDS with a
// 1152-entry index row): more independent work-groups in flight beat a
// deeper ring per work-group (at the 32K prefill 8.4 ms with two stages,
// 9.3 ms with three, 12.6 ms with four, 23.8 ms with five). The PV operand
// V^T comes from LDS through gfx950's transposing reads (two 8-byte reads
// per operand) instead of 16-byte reads and an 8 x 8 transpose in
// registers (32K prefill 6.58 -> 6.36 ms, 1M chunk 8.83 -> 7.91 ms).
#include "hs2_device.h"
#include "hs2_launch.h"

#include <type_traits>

namespace hs2 {

namespace {

constexpr int D = 128;
constexpr int TK = 32;                       // keys per tile
constexpr int HALF = TK * D * 2;             // 8 KB: K (or V) rows of a tile
constexpr int TILE_BYTES = 2 * HALF;
constexpr int NS = 2;                        // ring stages (see the kernel comment)
constexpr float RESCALE_GAP = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;

struct Sp2Args {
  const __bf16* q; const __bf16* k; const __bf16* v;
  const int32_t* idx;
  __bf16* o;
  int L, B, n_q, n_kv, h_q, h_kv, W;
  float c;
  KvRows kv;
  size_t layer_stride;  // elements between layers of q and o
};

// K rows are 256 B (16 chunks); a 16-byte read of 64 lanes is served 32
// lanes at a time from 128 banks (512 B), so rows of equal parity share
// banks. Swapping bits 0 and 2 of the row's low four bits in the swizzle
// puts the 32 chunks a half wave reads (lane groups 0-1 or 2-3, one row per
// l16) on distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return (row & 10) | ((row & 1) << 2) | ((row >> 2) & 1); }

// The many-query kernel keeps the 32-byte chunk pairs of its V rows
// XOR-swizzled by y = (key mod 8) ^ bit 3 of the tile key, so that its
// transposing reads (16 keys x 32 bytes per instruction) are free of bank
// conflicts whether the LDS serves them 64 lanes at a time from 128 banks
// (the eight keys of each parity get distinct y) or 32 lanes at a time from
// 64 banks (each run of eight consecutive keys gets distinct y); with
// y = bits 1-3 of the key the counters showed conflicts on 14 % of the
// pass's cycles.
__device__ __forceinline__ int vswz(int key) { return ((key & 7) ^ ((key >> 3) & 1)) << 1; }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// The P^T operand of lane group grp holds keys 4 grp + 0..3 and
// 16 + 4 grp + 0..3 of a 32-key tile. The matching V^T operand of head-dim
// block db comes straight from LDS with two transposing reads
// (ds_read_b64_tr_b16 gives lane 4a + b of each 16-lane group element b of
// the 8-byte pieces addressed by lanes a, a + 4, a + 8 and a + 12): lane
// a + 4c addresses head-dim elements 16 db + 4a .. + 3 of key 4 grp + c
// (then of key 16 + 4 grp + c), so lane l16 receives head-dim row
// 16 db + l16 of its group's eight keys. v_lane_offsets gives a lane's byte
// offsets of its two pieces for every db, relative to the tile's V rows.
__device__ __forceinline__ void v_lane_offsets(int grp, int l16, int (&o1)[8], int (&o2)[8]) {
  const int a = l16 & 3, c = l16 >> 2;
  const int k1 = 4 * grp + c, k2 = 16 + 4 * grp + c;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int chunk = 2 * db + (a >> 1);
    o1[db] = k1 * 256 + ((chunk ^ vswz(k1)) << 4) + ((a & 1) << 3);
    o2[db] = k2 * 256 + ((chunk ^ vswz(k2)) << 4) + ((a & 1) << 3);
  }
}
typedef __attribute__((address_space(3))) const char lds_cchar;
// the two pieces at LDS addresses p1 and p2
__device__ __forceinline__ bf16x8 v_operand(lds_cchar* p1, lds_cchar* p2) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p2);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (other counters untouched)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// wait until at most K * L_ of this wave's vector-memory operations are
// outstanding, for the run-time `ahead` in 0 .. K (the immediate must be a
// constant)
template <int K, int L_>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (K < 0) {
    return;
  } else {
    if (ahead == K) __builtin_amdgcn_s_waitcnt(vmcnt_imm(K * L_));
    else wait_ahead<K - 1, L_>(ahead);
  }
}

}  // namespace

// Index-row slots in LDS: the row padded to whole tiles, then one slot for
// the count of valid entries and three of padding (16-byte multiple).
__host__ __device__ constexpr int idx_row_slots(int width) { return (width + TK - 1) / TK * TK + 4; }

// Copies one index row (ascending, -1 padded) into LDS as K/V buffer rows,
// every slot past the valid entries (up to whole tiles) holding the first
// row, so the gather loop reads it unguarded; the slot after the padded row
// receives the number of valid entries (written by the one thread that holds
// the last valid entry, or by thread 0 when there is none).
template <int NTHREADS>
__device__ __forceinline__ int stage_index_row(const int32_t* irow, int W, int b, const KvRows& kv, int* sidx) {
  const int w_pad = (W + TK - 1) / TK * TK;
  const int j_first = W > 0 ? irow[0] : -1;
  const int first_row = j_first >= 0 ? (int)kv.row(b, j_first) : 0;
  if (threadIdx.x == 0 && j_first < 0) sidx[w_pad] = 0;
  for (int t = threadIdx.x; t < w_pad; t += NTHREADS) {
    const int j = t < W ? irow[t] : -1;
    sidx[t] = j >= 0 ? (int)kv.row(b, j) : first_row;
    if (j >= 0 && (t + 1 == W || irow[t + 1] < 0)) sidx[w_pad] = t + 1;
  }
  __syncthreads();
  return sidx[w_pad];
}

// NWV waves; wave w gathers keys [w*32/NWV, (w+1)*32/NWV) of every tile (K
// and V) and computes row block w.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void sparse_bf16_kernel(Sp2Args a) {
  using OP = Op<__bf16, D>;
  constexpr int KPW = TK / NWV;              // keys gathered per wave per tile
  constexpr int IPW = KPW / 4;               // 1 KB load instructions per half
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS targets stay scalar
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int rows_total = a.L * G;

  // KV head slowest: consecutive ids (one XCD, through the swizzle) are
  // neighbouring queries of one KV head, whose gathers overlap, so an XCD's
  // L2 holds one head's rows instead of every head's (32K prefill 8.4 ->
  // 7.1 ms, 1M chunk 9.6 -> 9.1 ms)
  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nbq = a.B * a.n_q;
  const int g = wg / nbq;
  const int bi = wg - g * nbq;                // b * n_q + i
  const int b = bi / a.n_q;
  const int i = bi - b * a.n_q;
  const int32_t* irow = a.idx + (size_t)bi * a.W;

  // the index row lives in LDS after the ring, so reading it in the loop
  // never waits on the gathers in flight
  // (entries become K/V buffer rows here: contiguous or through the page table)
  int* sidx = reinterpret_cast<int*>(smem + NS * TILE_BYTES);
  const int n_valid = stage_index_row<64 * NWV>(irow, a.W, b, a.kv, sidx);
  const int n_tiles = (n_valid + TK - 1) / TK;

  // the 16-byte chunk a lane moves in gather instruction j, as an address in
  // buffer row 0 (K chunks and V chunk pairs swizzled for the reads); a
  // gather adds the row's byte offset (32-bit row times row bytes)
  const uint32_t row_bytes = (uint32_t)a.h_kv * D * 2;
  const char* ksrc[IPW];
  const char* vsrc[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int key = wave * KPW + j * 4 + grp;          // tile-local key of this lane
    ksrc[j] = reinterpret_cast<const char*>(a.k + (size_t)g * D) + ((l16 ^ kswz(key)) << 4);
    vsrc[j] = reinterpret_cast<const char*>(a.v + (size_t)g * D) + ((l16 ^ vswz(key)) << 4);
  }

  // index entries of the lane's keys in the next tile to gather
  int nidx[IPW];
  auto read_idx = [&](int t) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) nidx[j] = sidx[t * TK + wave * KPW + j * 4 + grp];
  };
  auto issue = [&](int stage) {
    char* base = smem + stage * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const uint64_t off = (uint64_t)(uint32_t)nidx[j] * row_bytes;
      const int slot_base = (wave * KPW + j * 4) * 16;  // first 16-byte slot of the instruction
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(ksrc[j] + off),
                                       (lds_void*)(base + slot_base * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(vsrc[j] + off),
                                       (lds_void*)(base + HALF + slot_base * 16), 16, 0, 0);
    }
  };

  // this wave's rows: (layer, head-of-group) pairs rb*16 + l16
  const int r = wave * 16 + l16;
  const bool wave_active = wave * 16 < rows_total;
  Frag<__bf16, D> qf;
  if (r < rows_total) {
    const int layer = r / G, hh = r - (r / G) * G;
    load_slice<__bf16, D>(qf, a.q + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D),
                          lane);
  } else {
    zero_slice<__bf16, D>(qf);
  }
  float m_run = -1e30f, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // each lane's LDS addresses in ring stage 0: its four K-fragment chunks
  // of key block 0 and its V^T pieces of every head-dim block (a tile's
  // stage and key block only add constants, which fold into the reads)
  lds_cchar* lsm = (lds_cchar*)smem;
  lds_cchar* kp[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kp[u] = lsm + l16 * 256 + (((4 * grp + u) ^ kswz(l16)) << 4);
  lds_cchar* vp1[8];
  lds_cchar* vp2[8];
  {
    int vo1[8], vo2[8];
    v_lane_offsets(grp, l16, vo1, vo2);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      vp1[db] = lsm + HALF + vo1[db];
      vp2[db] = lsm + HALF + vo2[db];
      // opaque from here on: kept in registers, not recomputed per tile
      asm volatile("" : "+v"(vp1[db]), "+v"(vp2[db]));
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(kp[u]));

  // prologue: tiles 0 .. NS-2 in flight
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    if (t < n_tiles) {
      read_idx(t);
      issue(t);
    }
  }
  if (NS - 1 < n_tiles) read_idx(NS - 1);

  // one tile; the loop below runs tiles in pairs so that each one's ring
  // stage is a constant (its LDS offsets become instruction immediates)
  static_assert(NS == 2, "tiles alternate between two ring stages");
  auto tile = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_c)::value;
    // own loads of tile t done, then all waves'
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (t + 1 < n_tiles) {
      issue(ST ^ 1);
      if (t + 2 < n_tiles) read_idx(t + 2);
    }
    if (!wave_active) return;

    // K rows kb * 16 + l16 share the swizzle of l16, so key block kb sits a
    // constant 4 KB past block 0
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            kp[u] + ST * TILE_BYTES + kb * 4096);
        x = OP::mma(kf, qf.u[u], x);
      }
      s[kb] = x;
    }

    const int kbase = t * TK;
    if (kbase + TK > n_valid) {                         // the last tile: keys past the list
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kbase + kb * 16 + 4 * grp + e >= n_valid) s[kb][e] = -INFINITY;
    }
    const float tmax = row_group_max(max2f(max3f(s[0][0], s[0][1], s[0][2]),
                                           max3f(s[0][3], max3f(s[1][0], s[1][1], s[1][2]), s[1][3])));
    const float m_tile = tmax * a.c;
    const bool grow = m_tile > m_run + RESCALE_GAP;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? m_tile : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    float psum = 0.f;
    bf16x8 pu;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = fast_exp2(fmaf(s[kb][e], a.c, -m_run));
        psum += pe;
        pu[kb * 4 + e] = (__bf16)pe;
      }
    l_run += psum;

    // O^T += V^T . P^T, V^T read transposed from LDS
#pragma unroll
    for (int db = 0; db < 8; ++db)
      acc[db] = OP::mma(v_operand(vp1[db] + ST * TILE_BYTES, vp2[db] + ST * TILE_BYTES), pu, acc[db]);
  };
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    tile(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < n_tiles) tile(t, std::integral_constant<int, 0>{});

  if (r >= rows_total) return;
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int layer = r / G, hh = r - (r / G) * G;
  // lane (grp, l16) holds head-dim elements 16 db + 4 grp .. + 3 of its row
  __bf16* orow = a.o + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D) + grp * 4;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    bf16x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][e] * inv);
    *reinterpret_cast<bf16x4*>(orow + db * 16) = w;
  }
}

// Decode-shaped calls (few index lists, fewer work-groups than the chip
// holds): one work-group serves one (sequence, query, KV head) list with NP
// key partitions. Each partition is a group of NWV row-block waves with its
// own two-stage ring over a contiguous NP-th of the list's tiles, so NP
// tiles' gathers are in flight per work-group instead of one. At the end
// the partitions' online-softmax states (maximum, sum, O^T) go through LDS
// and the first partition's waves merge them in partition order, so the
// result does not depend on timing.
// (three partitions of three stages, or two of four, keep more tiles in
// flight per partition but measured the same on the 64 x 128K decode: the
// gathers, not their latency, set the time). V^T is transposed in
// registers here: the many-query kernel's transposing LDS reads measured
// about 2 % slower in this kernel.
constexpr int NP = 4;
constexpr int NSS = 2;
constexpr size_t SPLIT_RING_BYTES = (size_t)NP * NSS * TILE_BYTES;   // 128 KB

template <int NWV>
__global__ __launch_bounds__(64 * NWV * NP) void sparse_bf16_split_kernel(Sp2Args a) {
  using OP = Op<__bf16, D>;
  constexpr int KPW = TK / NWV;              // keys gathered per wave per tile
  constexpr int IPW = KPW / 4;               // 1 KB load instructions per half
  constexpr int LPW = 2 * IPW;               // load instructions per wave per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wid / NWV;                // key partition
  const int wave = wid - part * NWV;         // row block (and gather share) within it
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int rows_total = a.L * G;

  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nbq = a.B * a.n_q;
  const int g = wg / nbq;
  const int bi = wg - g * nbq;                // b * n_q + i
  const int b = bi / a.n_q;
  const int i = bi - b * a.n_q;
  const int32_t* irow = a.idx + (size_t)bi * a.W;

  // the index row (as K/V buffer rows) after the rings
  int* sidx = reinterpret_cast<int*>(smem + SPLIT_RING_BYTES);
  const int n_valid = stage_index_row<64 * NWV * NP>(irow, a.W, b, a.kv, sidx);
  const int n_tiles = (n_valid + TK - 1) / TK;
  // this partition's tiles [t_lo, t_lo + n_mine); every wave runs `steps`
  // barrier steps, the largest partition's tile count
  const int t_lo = n_tiles * part / NP;
  const int n_mine = n_tiles * (part + 1) / NP - t_lo;
  const int steps = (n_tiles + NP - 1) / NP;

  char* ring = smem + (size_t)part * NSS * TILE_BYTES;
  // the chunk a lane moves in gather instruction j, as an address in buffer
  // row 0; a gather adds the row's byte offset
  const uint32_t row_bytes = (uint32_t)a.h_kv * D * 2;
  const char* ksrc[IPW];
  const char* vsrc[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int key = wave * KPW + j * 4 + grp;          // tile-local key of this lane
    ksrc[j] = reinterpret_cast<const char*>(a.k + (size_t)g * D) + ((l16 ^ kswz(key)) << 4);
    vsrc[j] = reinterpret_cast<const char*>(a.v + (size_t)g * D) + (l16 << 4);
  }

  int nidx[IPW];
  auto read_idx = [&](int t) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) nidx[j] = sidx[(t_lo + t) * TK + wave * KPW + j * 4 + grp];
  };
  auto issue = [&](int stage) {
    char* base = ring + stage * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const uint64_t off = (uint64_t)(uint32_t)nidx[j] * row_bytes;
      const int slot_base = (wave * KPW + j * 4) * 16;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(ksrc[j] + off),
                                       (lds_void*)(base + slot_base * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(vsrc[j] + off),
                                       (lds_void*)(base + HALF + slot_base * 16), 16, 0, 0);
    }
  };

  const int r = wave * 16 + l16;
  const bool wave_active = wave * 16 < rows_total;
  Frag<__bf16, D> qf;
  if (r < rows_total) {
    const int layer = r / G, hh = r - (r / G) * G;
    load_slice<__bf16, D>(qf, a.q + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D),
                          lane);
  } else {
    zero_slice<__bf16, D>(qf);
  }
  float m_run = -1e30f, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: tiles 0 .. NSS-2 in flight
#pragma unroll
  for (int t = 0; t < NSS - 1; ++t) {
    if (t < n_mine) {
      read_idx(t);
      issue(t);
    }
  }
  if (NSS - 1 < n_mine) read_idx(NSS - 1);

  for (int t = 0; t < steps; ++t) {
    // own loads of tile t done (later tiles may stay in flight), then all waves'
    const int ahead = max(0, min(NSS - 2, n_mine - 1 - t));
    static_assert((NSS - 2) * LPW <= 63, "vmcnt range");
    wait_ahead<NSS - 2, LPW>(ahead);
    __syncthreads();
    if (t + NSS - 1 < n_mine) {
      issue((t + NSS - 1) % NSS);
      if (t + NSS < n_mine) read_idx(t + NSS);
    }
    if (t >= n_mine || !wave_active) continue;
    const char* base = ring + (t % NSS) * TILE_BYTES;

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kb * 16 + l16;
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(base + key * 256 + (((4 * grp + u) ^ kswz(key)) << 4));
        x = OP::mma(kf, qf.u[u], x);
      }
      s[kb] = x;
    }
    bf16x8 vraw[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int key = sl < 4 ? 4 * grp + sl : 16 + 4 * grp + (sl - 4);
      vraw[sl] = *reinterpret_cast<const bf16x8*>(base + HALF + key * 256 + l16 * 16);
    }

    const int kbase = (t_lo + t) * TK;
    if (kbase + TK > n_valid) {                         // the last tile: keys past the list
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kbase + kb * 16 + 4 * grp + e >= n_valid) s[kb][e] = -INFINITY;
    }
    const float tmax = row_group_max(max2f(max3f(s[0][0], s[0][1], s[0][2]),
                                           max3f(s[0][3], max3f(s[1][0], s[1][1], s[1][2]), s[1][3])));
    const float m_tile = tmax * a.c;
    const bool grow = m_tile > m_run + RESCALE_GAP;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? m_tile : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    float psum = 0.f;
    bf16x8 pu;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = fast_exp2(fmaf(s[kb][e], a.c, -m_run));
        psum += pe;
        pu[kb * 4 + e] = (__bf16)pe;
      }
    l_run += psum;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      bf16x8 vu;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) vu[sl] = vraw[sl][db];
      acc[db] = OP::mma(vu, pu, acc[db]);
    }
  }

  // merge: every partition's state into LDS (the rings are free after this
  // barrier), then the first partition's waves combine them in order
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);           // [NP][NWV][32][64] partial O^T
  float* mm = mo + NP * NWV * 32 * 64;                  // [NP][NWV][16] row maxima
  float* ml = mm + NP * NWV * 16;                       // [NP][NWV][16] row sums
  const int slot = part * NWV + wave;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo[(slot * 32 + db * 4 + e) * 64 + lane] = acc[db][e];
  if (grp == 0) {
    mm[slot * 16 + l16] = m_run;
    ml[slot * 16 + l16] = l;
  }
  __syncthreads();
  if (part != 0 || r >= rows_total) return;
  float M = -1e30f;
#pragma unroll
  for (int p = 0; p < NP; ++p) M = fmaxf(M, mm[(p * NWV + wave) * 16 + l16]);
  float L = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sp = p * NWV + wave;
    const float w = fast_exp2(mm[sp * 16 + l16] - M);
    L += ml[sp * 16 + l16] * w;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[db][e] += mo[(sp * 32 + db * 4 + e) * 64 + lane] * w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int layer = r / G, hh = r - (r / G) * G;
  __bf16* orow = a.o + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D) + grp * 32;
  bf16x8 outv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int db = 0; db < 8; ++db) outv[e][db] = (__bf16)(o[db][e] * inv);
#pragma unroll
  for (int e = 0; e < 4; ++e) reinterpret_cast<bf16x8*>(orow)[e] = outv[e];
}

// Dynamic LDS of one work-group: the ring plus the index row. Wider index
// rows than fit the default 64 KB per work-group (more than 8192 entries)
// go to the generic kernel, which keeps no index row in LDS.
constexpr size_t SPARSE_LDS_LIMIT = 64 * 1024;

size_t sparse_bf16_lds_bytes(int width) { return (size_t)NS * TILE_BYTES + (size_t)idx_row_slots(width) * sizeof(int); }

bool sparse_uses_bf16_kernel(const SparsePlan& p) {
  return p.bf16 && p.head_dim == D && (size_t)p.batch * p.n_q * p.h_kv >= 2048 &&
         p.layers * (p.h_q / p.h_kv) <= 64 && sparse_bf16_lds_bytes(p.width) <= SPARSE_LDS_LIMIT;
}

// The decode-shaped kernel needs the NP rings plus the index row, and after
// the loop the partitions' states; at most a work-group's 160 KB.
constexpr size_t SPLIT_LDS_LIMIT = 160 * 1024;

static size_t sparse_bf16_split_lds_bytes(int width, int nwv) {
  const size_t merge = (size_t)NP * nwv * (32 * 64 + 2 * 16) * sizeof(float);
  const size_t ring = SPLIT_RING_BYTES + (size_t)idx_row_slots(width) * sizeof(int);
  return ring > merge ? ring : merge;
}

bool sparse_uses_bf16_split_kernel(const SparsePlan& p) {
  const int rows = p.layers * (p.h_q / p.h_kv);
  return p.bf16 && p.head_dim == D && (size_t)p.batch * p.n_q * p.h_kv < 2048 && rows <= 32 &&
         sparse_bf16_split_lds_bytes(p.width, rows <= 16 ? 1 : 2) <= SPLIT_LDS_LIMIT;
}

hipError_t launch_sparse_attn_bf16(const SparsePlan& p, hipStream_t st) {
  Sp2Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.idx = p.idx;
  a.o = reinterpret_cast<__bf16*>(p.o);
  a.L = p.layers; a.B = p.batch; a.n_q = p.n_q; a.n_kv = p.n_kv;
  a.h_q = p.h_q; a.h_kv = p.h_kv; a.W = p.width; a.c = p.scale_log2; a.kv = p.kv;
  a.layer_stride = p.layer_stride ? p.layer_stride : (size_t)p.batch * p.n_q * p.h_q * D;
  const int G = p.h_q / p.h_kv;
  const int rb = (p.layers * G + 15) / 16;
  const dim3 grid((unsigned)((size_t)p.batch * p.n_q * p.h_kv));
  const size_t smem = sparse_bf16_lds_bytes(p.width);
  if (smem > SPARSE_LDS_LIMIT) return hipErrorInvalidValue;
  if (rb <= 1) hipLaunchKernelGGL(sparse_bf16_kernel<1>, grid, dim3(64), smem, st, a);
  else if (rb <= 2) hipLaunchKernelGGL(sparse_bf16_kernel<2>, grid, dim3(128), smem, st, a);
  else if (rb <= 4) hipLaunchKernelGGL(sparse_bf16_kernel<4>, grid, dim3(256), smem, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_sparse_attn_bf16_split(const SparsePlan& p, hipStream_t st) {
  Sp2Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.idx = p.idx;
  a.o = reinterpret_cast<__bf16*>(p.o);
  a.L = p.layers; a.B = p.batch; a.n_q = p.n_q; a.n_kv = p.n_kv;
  a.h_q = p.h_q; a.h_kv = p.h_kv; a.W = p.width; a.c = p.scale_log2; a.kv = p.kv;
  a.layer_stride = p.layer_stride ? p.layer_stride : (size_t)p.batch * p.n_q * p.h_q * D;
  const int rows = p.layers * (p.h_q / p.h_kv);
  const dim3 grid((unsigned)((size_t)p.batch * p.n_q * p.h_kv));
  if (grid.x == 0) return hipSuccess;
  struct Split1Tag {};
  struct Split2Tag {};
  if (rows <= 16) {
    const size_t smem = sparse_bf16_split_lds_bytes(p.width, 1);
    if (smem > SPLIT_LDS_LIMIT) return hipErrorInvalidValue;
    const hipError_t e = ensure_dynamic_lds<Split1Tag>((const void*)sparse_bf16_split_kernel<1>, (int)SPLIT_LDS_LIMIT);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_bf16_split_kernel<1>, grid, dim3(64 * NP), smem, st, a);
  } else if (rows <= 32) {
    const size_t smem = sparse_bf16_split_lds_bytes(p.width, 2);
    if (smem > SPLIT_LDS_LIMIT) return hipErrorInvalidValue;
    const hipError_t e = ensure_dynamic_lds<Split2Tag>((const void*)sparse_bf16_split_kernel<2>, (int)SPLIT_LDS_LIMIT);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_bf16_split_kernel<2>, grid, dim3(128 * NP), smem, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hs2
