// KV Bridging: each Cross-Decoder full layer's K and V are projections of
// the hidden states of its Self-Decoder full layer (HySparse2 pages:
// blog.lynxflow.co, section "Architectural Innovation: Two-Level KV
// Sharing"; hitechexpert.top, section "Two-Level KV Sharing"). This kernel
// writes them straight into the K/V buffers the Hybrid Block reads:
//   K[m, :] = hidden[m, :] . W_k^T,  V[m, :] = hidden[m, :] . W_v^T,
// with m running over all B * n tokens and W in the linear-layer layout
// [out features][d_model]. bf16 operands, fp32 accumulation, bf16 results.
//
// One GEMM C[M, 2F] = H[M, Dm] . W[2F, Dm]^T (F = h_kv * head_dim), computed
// transposed, C^T = W . H^T, so each lane ends up holding four consecutive
// output features of one token (8-byte stores along a K or V row). A
// work-group owns a 256-token x 256-feature block with eight waves, two per
// SIMD: a single wave per SIMD issues MFMAs at only about half the matrix
// core's rate, so the SIMD needs a second MFMA stream. Each wave computes a
// 128-token x 64-feature block (128 fp32 accumulators); every 16-byte H
// fragment it reads out of LDS feeds 4 MFMAs and every W fragment 8 (384 B
// of LDS reads per MFMA, under the LDS bandwidth at full MFMA rate). The
// 64-wide k-slices of H and W are staged by buffer loads straight into LDS,
// double-buffered, with a row swizzle that makes the fragment reads
// conflict-free.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

namespace {

constexpr int BM = 256;                     // tokens per work-group
constexpr int BN = 256;                     // output features per work-group
constexpr int BK = 64;                      // k-slice per stage
constexpr int ROW_BYTES = BK * 2;           // 128 B: one row of a slice
constexpr int SLICE_BYTES = BM * ROW_BYTES; // 32 KB (BM == BN)
constexpr int STAGE_BYTES = 2 * SLICE_BYTES;
constexpr int NSTAGE = 2;
constexpr int SMEM_BYTES = NSTAGE * STAGE_BYTES;

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk c of slice row r sits at chunk c ^ swz(r): the 16 rows a
// fragment read touches then cover all 64 banks once
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

struct BridgeArgs {
  const __bf16* h;      // [M][Dm]
  const __bf16* w;      // [2F][Dm]
  __bf16* k;            // [M][F]
  __bf16* v;            // [M][F]
  int M, F, Dm;
  int n_mt, n_nt;
};

}  // namespace

__global__ __launch_bounds__(512, 2) void kv_bridge_kernel(BridgeArgs a) {
  using OP = Op<__bf16, 128>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int wm = wave & 1, wn = wave >> 1;          // 2 x 4 waves of 128 x 64

  // feature tiles fastest: the tokens' slices are reused from L2 across them
  const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = lid % a.n_nt;
  const int mt = lid / a.n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int N = 2 * a.F;

  // stage the k-slice [kk, kk + 64) of the block's 256 token rows and 256
  // weight rows: 2 x 2048 chunks of 16 B, 4 of each per lane. Buffer loads
  // address them from one scalar resource per operand (the block's first
  // row) plus a 32-bit row/chunk offset per lane that the H and W slices
  // share; rows past the end of either matrix read as zeros.
  const int m_rows = min(BM, a.M - m0), n_rows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.h + (size_t)m0 * a.Dm), 0, m_rows * a.Dm * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w + (size_t)n0 * a.Dm), 0, n_rows * a.Dm * 2, 0x00020000);
  int voff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int slot = (wave * 4 + t) * 64 + lane;    // 0 .. 2047
    const int r = slot >> 3, pc = slot & 7;
    voff[t] = r * a.Dm * 2 + ((pc ^ swz(r)) << 4);
  }
  auto issue = [&](int kk, int stage) {
    char* base = smem + stage * STAGE_BYTES;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(hres, (lds_void*)(base + (wave * 4 + t) * 1024), 16,
                                               voff[t], kk * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres, (lds_void*)(base + SLICE_BYTES + (wave * 4 + t) * 1024), 16, voff[t], kk * 2, 0, 0);
    }
  };

  f32x4 acc[4][8];                                  // [feature block][token block]
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) acc[fb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment offsets: row (wave block + 16 * blk + l16), chunk 4u + grp;
  // rows 16 apart keep the same swizzle ((r >> 1) & 7 repeats every 16)
  const int hrow0 = wm * 128 + l16, wrow0 = wn * 64 + l16;
  int hoff[2], woff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    hoff[u] = hrow0 * ROW_BYTES + (((4 * u + grp) ^ swz(hrow0)) << 4);
    woff[u] = SLICE_BYTES + wrow0 * ROW_BYTES + (((4 * u + grp) ^ swz(wrow0)) << 4);
  }

  const int n_k = a.Dm / BK;
  issue(0, 0);
  for (int ks = 0; ks < n_k; ++ks) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ks + 1 < n_k) issue((ks + 1) * BK, (ks + 1) & 1);
    const char* base = smem + (ks & 1) * STAGE_BYTES;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // the k-substep's four W fragments stay in registers; the H
      // fragments stream one token block ahead of the MFMAs that use them
      bf16x8 wf[4], hf[2];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
        wf[fb] = *reinterpret_cast<const bf16x8*>(base + woff[u] + fb * 16 * ROW_BYTES);
      hf[0] = *reinterpret_cast<const bf16x8*>(base + hoff[u]);
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        if (tb + 1 < 8)
          hf[(tb + 1) & 1] = *reinterpret_cast<const bf16x8*>(base + hoff[u] + (tb + 1) * 16 * ROW_BYTES);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) acc[fb][tb] = OP::mma(wf[fb], hf[tb & 1], acc[fb][tb]);
      }
    }
  }

  // lane holds C^T[feature 4 * grp + i][token l16] of each 16 x 16 block
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) {
    const int m = m0 + wm * 128 + tb * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const int n = n0 + wn * 64 + fb * 16 + 4 * grp;
      if (n >= N) continue;
      __bf16* dst = n < a.F ? a.k + (size_t)m * a.F + n : a.v + (size_t)m * a.F + (n - a.F);
      __attribute__((ext_vector_type(4))) __bf16 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (__bf16)acc[fb][tb][e];
      *reinterpret_cast<decltype(w4)*>(dst) = w4;
    }
  }
}

hipError_t launch_kv_bridge(const BridgePlan& p, hipStream_t st) {
  BridgeArgs a;
  a.h = reinterpret_cast<const __bf16*>(p.hidden);
  a.w = reinterpret_cast<const __bf16*>(p.w_kv);
  a.k = reinterpret_cast<__bf16*>(p.k);
  a.v = reinterpret_cast<__bf16*>(p.v);
  a.M = p.tokens; a.F = p.features; a.Dm = p.d_model;
  a.n_mt = (a.M + BM - 1) / BM;
  a.n_nt = (2 * a.F + BN - 1) / BN;
  struct BridgeLdsTag {};
  {
    const hipError_t e = ensure_dynamic_lds<BridgeLdsTag>((const void*)kv_bridge_kernel, SMEM_BYTES);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((size_t)a.n_mt * a.n_nt));
  hipLaunchKernelGGL(kv_bridge_kernel, grid, dim3(512), SMEM_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace hs2
