// Backward pass of the full layer, for fine-tuning (HySparse2 pages:
// "Xiaomi Unveils HySparse2 for Faster Long-Context AI", section
// "Performance Gains: Cost, Speed, and Long-Context Capabilities": the
// models are fine-tuned before they are compared). Causal GQA softmax
// attention differentiated the usual way, with the forward's log-sum-exp:
//   P = 2^(t - lse2), t = logit * log2(e)      (lse2 = lse * log2(e))
//   dV += P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta = rowsum(dO * O)
//   dQ = scale dS K,  dK = scale dS^T Q
// Two kernels keep every sum in one place (no atomics, deterministic):
//   dK/dV: a work-group owns 16 keys per wave of one (sequence, KV head)
//          and walks every row (query, head of the group) that can see
//          them, 32 rows at a time staged in LDS; each wave keeps its keys'
//          dK^T and dV^T.
//   dQ:    a work-group owns 16 rows per wave, like the forward pass, and
//          walks the key tiles up to the causal limit, 64 keys at a time in
//          LDS.
// A third, small kernel forms Delta from O and dO.
//
// MFMA mapping (16x16 tiles, hs2_device.h). dK/dV kernel:
//   S = Q K^T, dP = dO V^T         A = row fragments (LDS), B = key rows (regs)
//   dV^T += dO^T P, dK^T += Q^T dS  A = dO^T / Q^T (LDS, transposed reads),
//                                   B = P / dS straight from the accumulators
// dQ kernel:
//   S^T = K Q^T, dP^T = V dO^T      A = key rows (LDS), B = row fragments (regs)
//   dQ^T += K^T dS^T                A = K^T (LDS, transposed reads), B = dS^T
// In both, a transposed operand's head-dim rows are permuted
// (d = DV * m + db, DV = D / 16) so that each lane reads one contiguous run
// of DV elements per row, and the contraction index (rows or keys) follows
// the accumulator layout: slot s of a lane maps to index
// (s < 4 ? 4*(l/16) + s : 16 + 4*(l/16) + s - 4).
#include <algorithm>

#include "hs2_bwd.h"
#include "hs2_device.h"
#include "hs2_launch.h"

// Work-group shapes (measured on the 32K prefill): dK/dV with one 16-key
// block per wave and eight waves (two per SIMD: 50 ms, against 56 ms for two
// blocks per wave at one wave per SIMD); dQ with one 16-row block per wave
// and eight waves.
#ifndef BWD_KB
#define BWD_KB 1
#endif
#ifndef BWD_NW
#define BWD_NW 8
#endif
#ifndef BWD_DQ_RBW
#define BWD_DQ_RBW 1
#endif
#ifndef BWD_DQ_NW
#define BWD_DQ_NW 8
#endif

namespace hs2 {

namespace {

constexpr float LOG2E = 1.4426950408889634f;

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;       // [B][h_q][n_q], natural log
  float* delta;           // [B][h_q][n_q]
  const void* acc_k;      // [B][n_kv][h_kv][D] sparse-layer sums, or NULL
  const void* acc_v;
  bool acc_fixed;         // 64-bit fixed point times acc_scale[2] (K), [3] (V)
  const float* acc_scale;
  void* dq; void* dk; void* dv;
  int B, n_q, n_kv, h_q, h_kv;
  int n_tiles;            // key tiles (dK/dV) or row tiles (dQ)
  float scale, scale_log2;
};

}  // namespace

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O): 16 lanes per (sequence, query, head) row
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int PER = D / 16;
  const size_t rows = (size_t)a.B * a.n_q * a.h_q;
  const size_t r = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float s = 0.f;
  if (r < rows) {
    const T* o = reinterpret_cast<const T*>(a.o) + r * D + sub * PER;
    const T* d = reinterpret_cast<const T*>(a.dout) + r * D + sub * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) s += to_f32(o[e]) * to_f32(d[e]);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
  if (r < rows && sub == 0) {
    // r = (b * n_q + i) * h_q + h  ->  [b][h][i]
    const int h = (int)(r % a.h_q);
    const size_t bi = r / a.h_q;
    const int i = (int)(bi % a.n_q);
    const int b = (int)(bi / a.n_q);
    a.delta[((size_t)b * a.h_q + h) * a.n_q + i] = s;
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* p, size_t n4) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n4; x += (size_t)gridDim.x * 256)
    p[x] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// dK, dV: KB 16-key blocks per wave, NW waves, rows in blocks of 32
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvSmem {
  static constexpr int LD = D + 16 / sizeof(T);
  T q[2][32][LD];
  T dout[2][32][LD];
  float lse2[2][32];
  float delta[2][32];
};

template <typename T, int D, int KB, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int DV = D / 16;
  constexpr int NT = 64 * NW;                         // threads
  constexpr int KT = NW * KB * 16;                    // keys per work-group
  constexpr int VEC = 16 / sizeof(T);
  constexpr int C16 = D / VEC;                        // 16-byte chunks per row
  constexpr int LOADS = (32 * C16 + NT - 1) / NT;     // per thread per tensor
  using SM = DkdvSmem<T, D>;
  __shared__ SM sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int R = a.n_q * G;
  const int q_off = a.n_kv - a.n_q;

  // longest first over the whole grid: key tile 0 (seen by the most rows)
  // of every (sequence, KV head), then tile 1, ...
  const int kt = (int)(blockIdx.x / (a.B * a.h_kv));
  const int bg = (int)(blockIdx.x % (a.B * a.h_kv));
  const int b = bg % a.B;
  const int g = bg / a.B;
  const int j0 = kt * KT;
  const int jw = j0 + wave * KB * 16;

  const T* qb = reinterpret_cast<const T*>(a.q);
  const T* db_ = reinterpret_cast<const T*>(a.dout);
  const size_t kstride = (size_t)a.h_kv * D;
  const T* kseq = reinterpret_cast<const T*>(a.k) + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const T* vseq = reinterpret_cast<const T*>(a.v) + ((size_t)b * a.n_kv * a.h_kv + g) * D;

  Frag<T, D> kf[KB], vf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = jw + kb * 16 + l16;
    if (j < a.n_kv) {
      load_slice<T, D>(kf[kb], kseq + (size_t)j * kstride, lane);
      load_slice<T, D>(vf[kb], vseq + (size_t)j * kstride, lane);
    } else {
      zero_slice<T, D>(kf[kb]);
      zero_slice<T, D>(vf[kb]);
    }
  }

  f32x4 dk[KB][DV], dv[KB][DV];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int d = 0; d < DV; ++d) {
      dk[kb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[kb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // rows that can see key j0: query positions >= j0
  const int r_begin = (max(0, j0 - q_off) * G) & ~31;
  const int n_rb = (R - r_begin + 31) / 32;

  uint4 qreg[LOADS], dreg[LOADS];
  float lreg = 0.f, dlreg = 0.f;
  auto gload = [&](int rbk) {
    const int r0 = r_begin + rbk * 32;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + NT * it;
      const int row = u / C16, c = u - (u / C16) * C16;
      const int r = r0 + row;
      if (row < 32 && r < R) {
        const int i = r / G, h = g * G + (r - (r / G) * G);
        const size_t off = (((size_t)b * a.n_q + i) * a.h_q + h) * D + c * VEC;
        qreg[it] = *reinterpret_cast<const uint4*>(qb + off);
        dreg[it] = *reinterpret_cast<const uint4*>(db_ + off);
      } else {
        qreg[it] = make_uint4(0, 0, 0, 0);
        dreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
    if (threadIdx.x < 32) {
      const int r = r0 + threadIdx.x;
      if (r < R) {
        const int i = r / G, h = g * G + (r - (r / G) * G);
        const size_t si = ((size_t)b * a.h_q + h) * a.n_q + i;
        lreg = a.lse[si] * LOG2E;
        dlreg = a.delta[si];
      } else {
        lreg = INFINITY;                              // P = 0 on padding rows
        dlreg = 0.f;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + NT * it;
      const int row = u / C16, c = u - (u / C16) * C16;
      if (row >= 32) break;
      *reinterpret_cast<uint4*>(&sm.q[buf][row][c * VEC]) = qreg[it];
      *reinterpret_cast<uint4*>(&sm.dout[buf][row][c * VEC]) = dreg[it];
    }
    if (threadIdx.x < 32) {
      sm.lse2[buf][threadIdx.x] = lreg;
      sm.delta[buf][threadIdx.x] = dlreg;
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int rbk = 0; rbk < n_rb; ++rbk) {
    const int buf = rbk & 1;
    if (rbk + 1 < n_rb) gload(rbk + 1);
    const int r0 = r_begin + rbk * 32;

    f32x4 p[2][KB], ds[2][KB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      Frag<T, D> qf, df;
      load_slice<T, D>(qf, &sm.q[buf][rb * 16 + l16][0], lane);
      load_slice<T, D>(df, &sm.dout[buf][rb * 16 + l16][0], lane);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        p[rb][kb] = dot_tile<T, D>(qf, kf[kb], f32x4{0.f, 0.f, 0.f, 0.f});
        ds[rb][kb] = dot_tile<T, D>(df, vf[kb], f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
    // lane holds rows 4*grp + e (of block rb), key l16 (of block kb)
    const bool need_mask = jw + KB * 16 - 1 > q_off + r0 / G;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rb * 16 + 4 * grp + e;
        const float l2 = sm.lse2[buf][row];
        const float dl = sm.delta[buf][row];
        const int pos = q_off + (r0 + row) / G;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          float x = fast_exp2(p[rb][kb][e] * a.scale_log2 - l2);
          if (need_mask && jw + kb * 16 + l16 > pos) x = 0.f;
          p[rb][kb][e] = x;
          ds[rb][kb][e] = x * (ds[rb][kb][e] - dl);
        }
      }

    TRows<T, D> tr;
    load_trows<T, D>(tr, &sm.dout[buf][0][0], SM::LD, lane);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) mma_t<T, D>(dv[kb], tr, p[0][kb], p[1][kb]);
    load_trows<T, D>(tr, &sm.q[buf][0][0], SM::LD, lane);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) mma_t<T, D>(dk[kb], tr, ds[0][kb], ds[1][kb]);

    if (rbk + 1 < n_rb) sstore(buf ^ 1);
    __syncthreads();
  }

  // lane holds dK^T / dV^T at d = DV*(4*grp + e) + db for key l16 of block kb
  T* dkb = reinterpret_cast<T*>(a.dk);
  T* dvb = reinterpret_cast<T*>(a.dv);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = jw + kb * 16 + l16;
    if (j >= a.n_kv) continue;
    const size_t off = (((size_t)b * a.n_kv + j) * a.h_kv + g) * D;
    const AccIn ak{a.acc_k, a.acc_fixed, a.acc_k && a.acc_fixed ? a.acc_scale[2] : 0.f};
    const AccIn av{a.acc_v, a.acc_fixed, a.acc_v && a.acc_fixed ? a.acc_scale[3] : 0.f};
    store_t_row<T, D>(dkb + off, dk[kb], a.scale, ak, off, grp);
    store_t_row<T, D>(dvb + off, dv[kb], 1.f, av, off, grp);
  }
}

// ---------------------------------------------------------------------------
// dQ: RBW 16-row blocks per wave, NW waves, key tiles of 64 in LDS
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqSmem {
  static constexpr int LD = D + 16 / sizeof(T);
  T k[2][64][LD];
  T v[2][64][LD];
};

template <typename T, int D, int RBW, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int DV = D / 16;
  constexpr int NT = 64 * NW;
  constexpr int ROWS = NW * RBW * 16;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int C16 = D / VEC;
  constexpr int LOADS = (64 * C16 + NT - 1) / NT;
  using SM = DqSmem<T, D>;
  __shared__ SM sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int R = a.n_q * G;
  const int q_off = a.n_kv - a.n_q;

  // longest first over the whole grid (row tile descending)
  const int rt = a.n_tiles - 1 - (int)(blockIdx.x / (a.B * a.h_kv));
  const int bg = (int)(blockIdx.x % (a.B * a.h_kv));
  const int b = bg % a.B;
  const int g = bg / a.B;
  const int r0 = rt * ROWS;
  const int i_hi = min(a.n_q - 1, (r0 + ROWS - 1) / G);
  const int n_kt = (q_off + i_hi + 64) / 64;

  const T* qb = reinterpret_cast<const T*>(a.q);
  const T* db_ = reinterpret_cast<const T*>(a.dout);
  const T* kseq = reinterpret_cast<const T*>(a.k) + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const T* vseq = reinterpret_cast<const T*>(a.v) + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const size_t kstride = (size_t)a.h_kv * D;

  Frag<T, D> qf[RBW], df[RBW];
  int row_pos[RBW];
  float l2[RBW], dl[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * RBW * 16 + rb * 16 + l16;
    if (r < R) {
      const int i = r / G, h = g * G + (r - (r / G) * G);
      const size_t off = (((size_t)b * a.n_q + i) * a.h_q + h) * D;
      load_slice<T, D>(qf[rb], qb + off, lane);
      load_slice<T, D>(df[rb], db_ + off, lane);
      const size_t si = ((size_t)b * a.h_q + h) * a.n_q + i;
      l2[rb] = a.lse[si] * LOG2E;
      dl[rb] = a.delta[si];
      row_pos[rb] = q_off + i;
    } else {
      zero_slice<T, D>(qf[rb]);
      zero_slice<T, D>(df[rb]);
      l2[rb] = INFINITY;
      dl[rb] = 0.f;
      row_pos[rb] = -1;
    }
  }

  f32x4 acc[RBW][DV];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int d = 0; d < DV; ++d) acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int tile) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + NT * it;
      const int row = u / C16, c = u - (u / C16) * C16;
      const int j = tile * 64 + row;
      if (row < 64 && j < a.n_kv) {
        kreg[it] = *reinterpret_cast<const uint4*>(kseq + (size_t)j * kstride + c * VEC);
        vreg[it] = *reinterpret_cast<const uint4*>(vseq + (size_t)j * kstride + c * VEC);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + NT * it;
      const int row = u / C16, c = u - (u / C16) * C16;
      if (row >= 64) break;
      *reinterpret_cast<uint4*>(&sm.k[buf][row][c * VEC]) = kreg[it];
      *reinterpret_cast<uint4*>(&sm.v[buf][row][c * VEC]) = vreg[it];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_kt) gload(t + 1);
    const int j0 = t * 64;
    const bool need_mask = j0 + 63 > q_off + r0 / G;

    f32x4 ds[4][RBW];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<T, D> kf, vf;
      load_slice<T, D>(kf, &sm.k[buf][kb * 16 + l16][0], lane);
      load_slice<T, D>(vf, &sm.v[buf][kb * 16 + l16][0], lane);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        const f32x4 s = dot_tile<T, D>(kf, qf[rb], f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 dp = dot_tile<T, D>(vf, df[rb], f32x4{0.f, 0.f, 0.f, 0.f});
        // lane holds keys 4*grp + e of block kb, row l16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = fast_exp2(s[e] * a.scale_log2 - l2[rb]);
          if (need_mask && j0 + kb * 16 + 4 * grp + e > row_pos[rb]) x = 0.f;
          ds[kb][rb][e] = x * (dp[e] - dl[rb]);
        }
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      TRows<T, D> tr;
      load_trows<T, D>(tr, &sm.k[buf][half * 32][0], SM::LD, lane);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        mma_t<T, D>(acc[rb], tr, ds[2 * half][rb], ds[2 * half + 1][rb]);
    }

    if (t + 1 < n_kt) sstore(buf ^ 1);
    __syncthreads();
  }

  T* dqb = reinterpret_cast<T*>(a.dq);
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * RBW * 16 + rb * 16 + l16;
    if (r >= R) continue;
    const int i = r / G, h = g * G + (r - (r / G) * G);
    store_t_row<T, D>(dqb + (((size_t)b * a.n_q + i) * a.h_q + h) * D, acc[rb], a.scale, AccIn{}, 0,
                      grp);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {

BwdArgs args_of(const BwdPlan& p) {
  BwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.dout = p.dout;
  a.lse = p.lse; a.delta = p.delta; a.acc_k = p.acc_k; a.acc_v = p.acc_v;
  a.acc_fixed = p.acc_fixed; a.acc_scale = p.acc_scale;
  a.dq = p.dq; a.dk = p.dk; a.dv = p.dv;
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.n_tiles = 0;
  a.scale = p.scale; a.scale_log2 = p.s.scale_log2;
  return a;
}

template <typename T, int D>
hipError_t launch_delta_t(const BwdPlan& p, hipStream_t st) {
  const BwdArgs a = args_of(p);
  const size_t rows = (size_t)a.B * a.n_q * a.h_q;
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dkdv_t(const BwdPlan& p, hipStream_t st) {
  BwdArgs a = args_of(p);
  constexpr int KB = BWD_KB, NW = BWD_NW;
  a.n_tiles = (a.n_kv + NW * KB * 16 - 1) / (NW * KB * 16);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, KB, NW>),
                     dim3((unsigned)((size_t)a.n_tiles * a.B * a.h_kv)), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dq_t(const BwdPlan& p, hipStream_t st) {
  BwdArgs a = args_of(p);
  constexpr int RBW = BWD_DQ_RBW, NW = BWD_DQ_NW;
  a.n_tiles = (a.n_q * (a.h_q / a.h_kv) + NW * RBW * 16 - 1) / (NW * RBW * 16);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, RBW, NW>),
                     dim3((unsigned)((size_t)a.n_tiles * a.B * a.h_kv)), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

// dispatch on (dtype, head_dim)
template <template <typename, int> class F>
hipError_t dispatch(const BwdPlan& p, hipStream_t st) {
  if (p.s.bf16) {
    if (p.s.head_dim == 128) return F<__bf16, 128>::run(p, st);
    if (p.s.head_dim == 64) return F<__bf16, 64>::run(p, st);
  } else {
    if (p.s.head_dim == 128) return F<float, 128>::run(p, st);
    if (p.s.head_dim == 64) return F<float, 64>::run(p, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
struct DeltaF { static hipError_t run(const BwdPlan& p, hipStream_t st) { return launch_delta_t<T, D>(p, st); } };
template <typename T, int D>
struct DkdvF { static hipError_t run(const BwdPlan& p, hipStream_t st) { return launch_dkdv_t<T, D>(p, st); } };
template <typename T, int D>
struct DqF { static hipError_t run(const BwdPlan& p, hipStream_t st) { return launch_dq_t<T, D>(p, st); } };

}  // namespace

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t n4 = n / 4;                        // callers pass multiples of 4
  const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const BwdPlan& p, hipStream_t st) { return dispatch<DeltaF>(p, st); }
hipError_t launch_bwd_dkdv_bf16(const BwdPlan& p, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdPlan& p, hipStream_t st) {
  if (p.qt && bwd_dq_uses_bf16_kernel(p.s)) return launch_bwd_dkdv_bf16(p, st);
  return dispatch<DkdvF>(p, st);
}
hipError_t launch_bwd_dq_bf16(const BwdPlan& p, hipStream_t st);

hipError_t launch_bwd_dq(const BwdPlan& p, hipStream_t st) {
  if (p.kt && bwd_dq_uses_bf16_kernel(p.s)) return launch_bwd_dq_bf16(p, st);
  return dispatch<DqF>(p, st);
}

}  // namespace hs2
