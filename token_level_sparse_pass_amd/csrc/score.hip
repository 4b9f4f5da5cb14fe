// Pass 2 of the full layer: the token-importance score. The full layer of a
// Hybrid Block "determines which tokens are important" (HySparse2 pages:
// openai-hub.net, section "From Hybrid SWA to HySparse2"); the score used is
// the layer's own softmax probability summed over every query head,
//   S(p, j) = sum_h 2^(t_h(p, j) - m2_h(p)) / l_h(p),   t = logit * log2(e),
// with (m2, l) the exact row statistics of pass 1, so the normaliser covers
// every key j <= p (window keys included).
//
// The head sum couples all query heads at each (query, key), so a
// work-group owns a 128-query x 256-key block of S and loops over all heads
// itself (fixed order, no atomics: the result is bit-reproducible). Each of
// the 8 waves keeps the K rows of its 64 keys in registers for the G heads
// that share them, reads Q of the current head from LDS (double-buffered),
// and keeps its 64x64 block of S in registers until every head is summed.
// Logits come from bf16 (or fp32) MFMA with fp32 accumulation.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

struct ScoreArgs {
  const void* q; const void* k;
  const float* stats;
  float* scores; size_t stride;
  int B, n_q, n_kv, h_q, h_kv;
  int b, q0, rows, window;
  int n_qt, n_kt;
  float scale_log2;
};

template <typename T, int D>
struct ScoreSmem {
  static constexpr int LD = D + 16 / sizeof(T);
  T q[2][128][LD];
  float m2[2][128];
  float il[2][128];
};

template <typename T, int D>
__global__ __launch_bounds__(512) void score_prefill_kernel(ScoreArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int V16_ROW = D / VEC;
  constexpr int QLOADS = 128 * V16_ROW / 512;
  __shared__ ScoreSmem<T, D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int wq = wave >> 2, wk = wave & 3;
  const int G = a.h_q / a.h_kv;
  const int q_off = a.n_kv - a.n_q;

  const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int qt = lid / a.n_kt;
  const int kt = lid - qt * a.n_kt;
  const int r_lo = qt * 128;                          // first row of the tile
  const int r_hi = min(a.rows, r_lo + 128) - 1;       // last valid row
  const int p_hi = q_off + a.q0 + r_hi;
  const int kj0 = kt * 256;
  if (kj0 > p_hi - a.window) return;                  // no candidate key here

  const T* qseq = reinterpret_cast<const T*>(a.q) + (size_t)a.b * a.n_q * a.h_q * D;
  const T* kseq = reinterpret_cast<const T*>(a.k) + (size_t)a.b * a.n_kv * a.h_kv * D;
  const size_t plane = (size_t)a.B * a.h_q * a.n_q;

  uint4 qreg[QLOADS];
  float st_reg = 0.f;
  auto gload_q = [&](int h) {
#pragma unroll
    for (int it = 0; it < QLOADS; ++it) {
      const int u = threadIdx.x + 512 * it;
      const int row = u / V16_ROW, c16 = u - (u / V16_ROW) * V16_ROW;
      const int r = r_lo + row;
      if (r < a.rows)
        qreg[it] = *reinterpret_cast<const uint4*>(
            qseq + ((size_t)(a.q0 + r) * a.h_q + h) * D + c16 * VEC);
      else
        qreg[it] = make_uint4(0, 0, 0, 0);
    }
    if (threadIdx.x < 256) {
      const int row = threadIdx.x & 127;
      const int r = r_lo + row;
      const size_t si = ((size_t)a.b * a.h_q + h) * a.n_q + a.q0 + min(r, a.rows - 1);
      st_reg = (threadIdx.x < 128) ? a.stats[si] : a.stats[plane + si];
    }
  };
  auto sstore_q = [&](int buf) {
#pragma unroll
    for (int it = 0; it < QLOADS; ++it) {
      const int u = threadIdx.x + 512 * it;
      const int row = u / V16_ROW, c16 = u - (u / V16_ROW) * V16_ROW;
      *reinterpret_cast<uint4*>(&sm.q[buf][row][c16 * VEC]) = qreg[it];
    }
    if (threadIdx.x < 128) sm.m2[buf][threadIdx.x] = st_reg;
    else if (threadIdx.x < 256) sm.il[buf][threadIdx.x - 128] = 1.f / st_reg;
  };

  f32x4 sacc[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload_q(0);
  sstore_q(0);
  __syncthreads();

  const int n_heads = a.h_q;
  Frag<T, D> kf[4];
  for (int h = 0; h < n_heads; ++h) {
    const int buf = h & 1;
    const int g = h / G;
    if (h - g * G == 0) {
      // K rows of this wave's 64 keys for KV head g, reused by its G heads
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int j = kj0 + wk * 64 + kb * 16 + (lane & 15);
        if (j < a.n_kv)
          load_slice<T, D>(kf[kb], kseq + ((size_t)j * a.h_kv + g) * D, lane);
        else
          zero_slice<T, D>(kf[kb]);
      }
    }
    if (h + 1 < n_heads) gload_q(h + 1);

#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int qrow = wq * 64 + qb * 16 + (lane & 15);
      Frag<T, D> qf;
      load_slice<T, D>(qf, &sm.q[buf][qrow][0], lane);
      const float m2 = sm.m2[buf][qrow];
      const float il = sm.il[buf][qrow];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 sv = dot_tile<T, D>(kf[kb], qf, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[qb][kb][e] = fmaf(fast_exp2(fmaf(sv[e], a.scale_log2, -m2)), il, sacc[qb][kb][e]);
      }
    }

    if (h + 1 < n_heads) sstore_q(buf ^ 1);
    __syncthreads();
  }

  // store: lane holds query (qb, lane%16) and 4 consecutive keys
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int r = r_lo + wq * 64 + qb * 16 + (lane & 15);
    if (r >= a.rows) continue;
    float* srow = a.scores + (size_t)r * a.stride;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int j = kj0 + wk * 64 + kb * 16 + 4 * grp;
      *reinterpret_cast<f32x4*>(srow + j) = sacc[qb][kb];
    }
  }
}

template <typename T, int D>
static hipError_t launch_score_t(const ScorePlan& p, hipStream_t st) {
  ScoreArgs a;
  a.q = p.q; a.k = p.k; a.stats = p.stats; a.scores = p.scores; a.stride = p.score_stride;
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.b = p.b; a.q0 = p.q0; a.rows = p.rows; a.window = p.window;
  a.scale_log2 = p.s.scale_log2;
  const int q_off = a.n_kv - a.n_q;
  const int n_cand_max = q_off + p.q0 + p.rows - 1 - p.window + 1;
  if (n_cand_max <= 0) return hipSuccess;
  a.n_qt = (p.rows + 127) / 128;
  a.n_kt = (n_cand_max + 255) / 256;
  const dim3 grid((unsigned)((size_t)a.n_qt * a.n_kt));
  hipLaunchKernelGGL((score_prefill_kernel<T, D>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_score_prefill_generic(const ScorePlan& p, hipStream_t st) {
  if (p.s.bf16) {
    if (p.s.head_dim == 128) return launch_score_t<__bf16, 128>(p, st);
    if (p.s.head_dim == 64) return launch_score_t<__bf16, 64>(p, st);
  } else {
    if (p.s.head_dim == 128) return launch_score_t<float, 128>(p, st);
    if (p.s.head_dim == 64) return launch_score_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hs2
