// Pass 1 of the full layer for decode-shaped calls (one query per
// sequence), specialised for bf16 and head dim 128: causal GQA attention of
// the query's heads over every cached key, split over the keys (split-KV),
// with every logit stored for the score pass (HySparse2 pages: openai-hub.net,
// section "From Hybrid SWA to HySparse2": the full layer computes attention
// and decides which tokens matter; hitechexpert.top, section "Two-Level KV
// Sharing": the sparse layers reuse this layer's KV cache).
//
// Decode streams K and V once at 8 flop per byte, so the kernel is built to
// keep HBM busy: one wave per (sequence, KV head, key split) gathers 32-key
// tiles of K and V straight into a 5-stage LDS ring (global_load_lds, four
// tiles in flight while one is used), so no load ever waits in a register.
// The G query heads of the KV head form one 16-row MFMA block:
// logits^T = K.Q^T and O^T += V^T.P^T with P taken from the accumulator.
// Each split leaves a partial record (m2, l, unnormalised O) that the
// combine step of attn_fwd.hip merges; the raw logits (q.k, before the
// softmax scale) go to the workspace, where the decode score step reads
// them instead of reading K a second time.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

namespace {

constexpr int D = 128;
constexpr int TK = 32;                       // keys per tile
constexpr int HALF = TK * D * 2;             // 8 KB: K (or V) rows of a tile
constexpr int TILE_BYTES = 2 * HALF;
constexpr int NS = 5;                        // ring stages
constexpr int LPT = 2 * TK / 4;              // 1 KB load instructions per tile (K and V)
constexpr float RESCALE_GAP = 8.0f;          // log2 units

typedef __attribute__((address_space(3))) void lds_void;

struct Dec2Args {
  const __bf16* q; const __bf16* k; const __bf16* v;
  float* part; float* logits; size_t lstride;
  const int32_t* seq_len;
  KvRows kv;
  int B, n_kv, h_q, h_kv, kps, n_split;
  float c;                                   // softmax scale * log2(e)
};

// K rows are 256 B (16 chunks); a 16-byte read of 64 lanes is served 32
// lanes at a time from 128 banks (512 B), so rows of equal parity share
// banks. Swapping bits 0 and 2 of the row's low four bits in the swizzle
// puts the 32 chunks a half wave reads (lane groups 0-1 or 2-3, one row per
// l16) on distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return (row & 10) | ((row & 1) << 2) | ((row >> 2) & 1); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (other counters untouched)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most n vector-memory operations of this wave are in flight
// (0 <= n <= 63). Vector memory operations of a wave complete in
// issue order on this architecture, so counting the loads and stores issued
// after a tile's loads turns this into "every load of that tile landed".
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define HS2_W(N) case N: __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); return;
    HS2_W(1) HS2_W(2) HS2_W(3) HS2_W(4) HS2_W(5) HS2_W(6) HS2_W(7) HS2_W(8)
    HS2_W(9) HS2_W(10) HS2_W(11) HS2_W(12) HS2_W(13) HS2_W(14) HS2_W(15) HS2_W(16)
    HS2_W(17) HS2_W(18) HS2_W(19) HS2_W(20) HS2_W(21) HS2_W(22) HS2_W(23) HS2_W(24)
    HS2_W(25) HS2_W(26) HS2_W(27) HS2_W(28) HS2_W(29) HS2_W(30) HS2_W(31) HS2_W(32)
    HS2_W(33) HS2_W(34) HS2_W(35) HS2_W(36) HS2_W(37) HS2_W(38) HS2_W(39) HS2_W(40)
    HS2_W(41) HS2_W(42) HS2_W(43) HS2_W(44) HS2_W(45) HS2_W(46) HS2_W(47) HS2_W(48)
    HS2_W(49) HS2_W(50) HS2_W(51) HS2_W(52) HS2_W(53) HS2_W(54) HS2_W(55) HS2_W(56)
    HS2_W(57) HS2_W(58) HS2_W(59) HS2_W(60) HS2_W(61) HS2_W(62) HS2_W(63)
#undef HS2_W
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); return;
  }
}

}  // namespace

__global__ __launch_bounds__(64) void attn_decode_bf16_kernel(Dec2Args a) {
  using OP = Op<__bf16, D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;

  // the KV heads of one key range are neighbours in launch order (and so
  // run together on one XCD): each key's rows of all KV heads share a
  // contiguous run of memory, which they then read at about the same time
  const uint32_t unit = xcd_swizzle(blockIdx.x, gridDim.x);
  const int g = unit % a.h_kv;
  const int bs = unit / a.h_kv;
  const int split = bs % a.n_split;
  const int b = bs / a.n_split;
  const int n_keys = a.seq_len ? a.seq_len[b] : a.n_kv;   // keys of this sequence
  const int k_begin = split * a.kps;
  const int k_end = min(n_keys, k_begin + a.kps);
  const int n_tiles = k_end > k_begin ? (k_end - k_begin + TK - 1) / TK : 0;

  const size_t kvs = (size_t)a.h_kv * D;
  const __bf16* kseq = a.k + (size_t)g * D;             // + row * kvs
  const __bf16* vseq = a.v + (size_t)g * D;

  // paged pool: lane i holds the id of the split's i-th page (a split spans
  // at most 64 pages of >= 32 rows); a 32-key tile never crosses a page
  const int first_page = a.kv.paged() ? (k_begin >> a.kv.page_shift) : 0;
  int page_id = 0;
  if (a.kv.paged() && first_page + lane < a.kv.max_pages && n_tiles > 0)
    page_id = a.kv.table[(size_t)b * a.kv.max_pages + first_page + lane];

  // tile t into ring stage `stage`: lane group grp of instruction j carries
  // key 4j + grp (clamped to the last key, whose rows are never used)
  auto issue = [&](int t, int stage) {
    char* base = smem + stage * TILE_BYTES;
    const int j0 = k_begin + t * TK;
    size_t row0;                                        // cache row of key j0
    if (a.kv.paged()) {
      const int pid = __builtin_amdgcn_readlane(page_id, (j0 >> a.kv.page_shift) - first_page);
      row0 = a.kv.page_row(pid, j0);
    } else {
      row0 = (size_t)b * a.n_kv + j0;
    }
#pragma unroll
    for (int j = 0; j < TK / 4; ++j) {
      const int key = j * 4 + grp;
      const size_t row = (row0 + (size_t)(min(j0 + key, k_end - 1) - j0)) * kvs;
      // K and V are read once: non-temporal (nt) loads, which leave the
      // caches to the logits this kernel writes and the score step reads
      // back (pass 1 3.67 -> 3.53 ms, score step 0.185 -> 0.173 ms at the
      // 64 x 128K decode)
      __builtin_amdgcn_global_load_lds(kseq + row + ((l16 ^ kswz(key)) << 3),
                                       (lds_void*)(base + j * 1024), 16, 0, 2);
      __builtin_amdgcn_global_load_lds(vseq + row + (l16 << 3),
                                       (lds_void*)(base + HALF + j * 1024), 16, 0, 2);
    }
  };

  // rows: the G query heads of KV head g (16-row block, unused rows zero)
  const int hh = l16;
  const bool row_ok = hh < G;
  Frag<__bf16, D> qf;
  if (row_ok) load_slice<__bf16, D>(qf, a.q + ((size_t)b * a.h_q + g * G + hh) * D, lane);
  else zero_slice<__bf16, D>(qf);
  // raw logits of this lane's query head: one row of lstride floats per
  // (sequence, head); lane (grp, hh) holds keys 4 grp .. 4 grp + 3 of each
  // 16-key block, so a tile leaves as two 16-byte stores per lane
  float* lgt = a.logits + ((size_t)b * a.h_q + g * G + min(l16, G - 1)) * a.lstride;
  constexpr int SPT = 2;                        // store instructions per tile

  float m_run = -1e30f, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < n_tiles) issue(t, t);

  for (int t = 0; t < n_tiles; ++t) {
    // tile t has landed once at most the later tiles' loads (issued after
    // it) and the logit stores of the tiles since are in flight
    static_assert(LPT * (NS - 2) + SPT * (NS - 1) <= 63, "vmcnt holds at most 63");
    wait_vm(LPT * min(NS - 2, n_tiles - 1 - t) + SPT * min(t, NS - 1));
    __syncthreads();
    // the stage refilled below was read in the previous iteration, whose
    // LDS reads all completed before their MFMAs could issue
    if (t + NS - 1 < n_tiles) issue(t + NS - 1, (t + NS - 1) % NS);
    const char* base = smem + (t % NS) * TILE_BYTES;

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
    // V rows of the lane's 8 key slots (k<4: 4g+k, k>=4: 16+4g+k-4), read
    // with the bf16 vector type so the compiler adds no wait on the ring
    bf16x8 vraw[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int key = sl < 4 ? 4 * grp + sl : 16 + 4 * grp + (sl - 4);
      vraw[sl] = *reinterpret_cast<const bf16x8*>(base + HALF + key * 256 + l16 * 16);
    }

    const int kbase = k_begin + t * TK;
    // raw logits of the valid heads for the score step (rows are padded to
    // whole tiles, and keys past the sequence's length are never read back);
    // lanes 0..G-1 of every lane group store, so each tile issues exactly
    // SPT store instructions
    if (row_ok) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        *reinterpret_cast<f32x4*>(lgt + kbase + kb * 16 + 4 * grp) = s[kb];
    }

    if (kbase + TK > k_end) {
      // the split's last tile: keys past its end take no weight
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kbase + kb * 16 + 4 * grp + e >= k_end) s[kb][e] = -INFINITY;
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

    // O^T += V^T . P^T: head-dim rows permuted so lane l reads V[key][8*l16..+7]
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      bf16x8 vu;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) vu[sl] = vraw[sl][db];
      acc[db] = OP::mma(vu, pu, acc[db]);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // partial record per (b, head, split): m2, l, O[d] (unnormalised); an
  // empty split leaves m2 = -1e30, l = 0, O = 0, which the combine weighs 0
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  float* rec = a.part + (((size_t)b * a.h_q + g * G + hh) * a.n_split + split) * (D + 2);
  if (grp == 0) {
    rec[0] = m_run;
    rec[1] = l;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int db = 0; db < 8; ++db) rec[2 + 8 * (4 * grp + e) + db] = acc[db][e];
}

bool decode_uses_bf16_kernel(const Shape& s) {
  return s.bf16 && s.head_dim == D && s.h_q / s.h_kv <= 16;
}

hipError_t launch_attn_decode_bf16(const DecodePlan& p, hipStream_t st) {
  Dec2Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.part = p.part; a.logits = p.logits; a.lstride = p.logits_stride; a.seq_len = p.seq_len;
  a.kv = p.kv;
  a.B = p.s.batch; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.kps = p.keys_per_split; a.n_split = p.n_split; a.c = p.s.scale_log2;
  const dim3 grid((unsigned)((size_t)a.B * a.h_kv * a.n_split));
  hipLaunchKernelGGL(attn_decode_bf16_kernel, grid, dim3(64), NS * TILE_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace hs2
