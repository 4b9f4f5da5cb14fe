// Sparse layers with KV Reuse, specialised for bf16 and head dim 128 on
// many queries (prefill-shaped calls). Same contract as sparse_attn.hip:
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
// 9.3 ms with three, 12.6 ms with four, 23.8 ms with five).
#include "hs2_device.h"
#include "hs2_launch.h"

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

__device__ __forceinline__ int kswz(int row) { return row & 15; }

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

// NWV waves; wave w gathers keys [w*32/NWV, (w+1)*32/NWV) of every tile (K
// and V) and computes row block w.
template <int NWV>
__global__ __launch_bounds__(64 * NWV) void sparse_bf16_kernel(Sp2Args a) {
  using OP = Op<__bf16, D>;
  constexpr int KPW = TK / NWV;              // keys gathered per wave per tile
  constexpr int IPW = KPW / 4;               // 1 KB load instructions per half
  constexpr int LPW = 2 * IPW;               // load instructions per wave per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int rows_total = a.L * G;

  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int g = wg % a.h_kv;
  const int bi = wg / a.h_kv;                 // b * n_q + i
  const int b = bi / a.n_q;
  const int i = bi - b * a.n_q;
  const int32_t* irow = a.idx + (size_t)bi * a.W;

  // the index row lives in LDS after the ring, so reading it in the loop
  // never waits on the gathers in flight
  // (entries become K/V buffer rows here: contiguous or through the page table)
  int* sidx = reinterpret_cast<int*>(smem + NS * TILE_BYTES);
  for (int t = threadIdx.x; t < a.W; t += 64 * NWV) {
    const int j = irow[t];
    sidx[t] = j >= 0 ? (int)a.kv.row(b, j) : -1;
  }
  __syncthreads();
  int n_valid = 0;
  for (int t = lane; t < a.W; t += 64) n_valid += (sidx[t] >= 0) ? 1 : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n_valid += __shfl_xor(n_valid, m, 64);
  const int n_tiles = (n_valid + TK - 1) / TK;
  const int fallback = n_valid > 0 ? sidx[0] : 0;

  const size_t kvs = (size_t)a.h_kv * D;
  const __bf16* kseq = a.k + (size_t)g * D;             // + buffer row * kvs
  const __bf16* vseq = a.v + (size_t)g * D;

  // index entries of the lane's keys in the next tile to gather
  int nidx[IPW];
  auto read_idx = [&](int t) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int pos = t * TK + wave * KPW + j * 4 + grp;
      nidx[j] = pos < n_valid ? sidx[pos] : fallback;
    }
  };
  auto issue = [&](int stage) {
    char* base = smem + stage * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int key = wave * KPW + j * 4 + grp;        // tile-local key of this lane
      const size_t row = (size_t)nidx[j] * kvs;
      const int slot_base = (wave * KPW + j * 4) * 16;  // first 16-byte slot of the instruction
      const int pc = l16;
      __builtin_amdgcn_global_load_lds(kseq + row + ((pc ^ kswz(key)) << 3),
                                       (lds_void*)(base + slot_base * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vseq + row + (pc << 3),
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

  // prologue: tiles 0 .. NS-2 in flight
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    if (t < n_tiles) {
      read_idx(t);
      issue(t);
    }
  }
  if (NS - 1 < n_tiles) read_idx(NS - 1);

  for (int t = 0; t < n_tiles; ++t) {
    // own loads of tile t done (later tiles may stay in flight), then all waves'
    const int ahead = min(NS - 2, n_tiles - 1 - t);
    static_assert((NS - 2) * LPW <= 63, "vmcnt range");
    wait_ahead<NS - 2, LPW>(ahead);
    __syncthreads();
    if (t + NS - 1 < n_tiles) {
      issue((t + NS - 1) % NS);
      if (t + NS < n_tiles) read_idx(t + NS);
    }
    if (!wave_active) continue;
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
    // V rows of the lane's 8 key slots (k<4: 4g+k, k>=4: 16+4g+k-4); read
    // with the bf16 vector type like every other LDS read here, which keeps
    // the compiler from adding a full wait on the gathers in flight
    bf16x8 vraw[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int key = sl < 4 ? 4 * grp + sl : 16 + 4 * grp + (sl - 4);
      vraw[sl] = *reinterpret_cast<const bf16x8*>(base + HALF + key * 256 + l16 * 16);
    }

    const int kbase = t * TK;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (kbase + kb * 16 + 4 * grp + e >= n_valid) s[kb][e] = -INFINITY;
        tmax = fmaxf(tmax, s[kb][e]);
      }
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
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

  if (r >= rows_total) return;
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int layer = r / G, hh = r - (r / G) * G;
  __bf16* orow = a.o + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D) + grp * 32;
  bf16x8 outv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int db = 0; db < 8; ++db) outv[e][db] = (__bf16)(acc[db][e] * inv);
#pragma unroll
  for (int e = 0; e < 4; ++e) reinterpret_cast<bf16x8*>(orow)[e] = outv[e];
}

bool sparse_uses_bf16_kernel(const SparsePlan& p) {
  return p.bf16 && p.head_dim == D && (size_t)p.batch * p.n_q * p.h_kv >= 2048;
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
  const size_t smem = NS * TILE_BYTES + (size_t)p.width * sizeof(int);
  if (rb <= 1) hipLaunchKernelGGL(sparse_bf16_kernel<1>, grid, dim3(64), smem, st, a);
  else if (rb <= 2) hipLaunchKernelGGL(sparse_bf16_kernel<2>, grid, dim3(128), smem, st, a);
  else if (rb <= 4) hipLaunchKernelGGL(sparse_bf16_kernel<4>, grid, dim3(256), smem, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hs2
