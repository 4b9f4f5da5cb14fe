// Backward pass of the sparse layers over their fixed index sets (KV Reuse:
// HySparse2 pages, "Xiaomi Unveils HySparse2 for Faster Long-Context AI",
// section "Two-Level KV Sharing": every sparse layer reads the full layer's
// K/V, so their K and V gradients all land in the same buffer; section
// "Performance Gains: Cost, Speed, and Long-Context Capabilities" for the
// fine-tuning that needs them).
//
// One work-group serves one (sequence b, query i, KV head g), like the
// forward kernel: its rows are all (layer, head of group g) pairs (at most
// 64), and the index list is walked in 32-key tiles. All eight waves first
// re-derive each row's log-sum-exp over the list. Then row waves 0..3 (one
// per 16 rows) compute, per tile,
//   S^T = K_sel Q^T, dP^T = V_sel dO^T, P^T = 2^(t - lse2),
//   dS^T = P^T (dP^T - Delta),  dQ^T += K_sel^T dS^T      (kept in registers)
// and put P^T and dS^T into LDS, while contraction waves 4..7 take the
// previous tile and contract over the rows:
//   dK_sel = scale dS^T Q,  dV_sel = P^T dO      (32 keys x D each)
// adding the results to accumulators [B][n_kv][h_kv][D] with atomics: a key
// appears in the index sets of many queries, and the accumulators are
// folded into dK and dV by the full layer's dK/dV kernel. The accumulators
// are fp32 (fastest; the order in which the adds land changes the last
// bits), or, for the deterministic entry point, 64-bit fixed point: each
// addend is rounded to a multiple of 2^-F, F from a bound on what any sum
// can reach (launch_sparse_bwd_bounds), and integer sums do not depend on
// the order of the adds. Their resolution (2^-39 for dV and 2^-34 for dK at
// the 32K prefill) is far finer than fp32 sums keep. Keeping the
// atomics on waves that issue no loads matters: a wave's vector memory
// operations complete in order, so a load issued after a burst of atomics
// would wait for all of them. Each atomic instruction covers four keys x 16
// consecutive floats (64-byte segments), the cheapest pattern measured.
//
// LDS tiles hold P^T and dS^T as [key][row], rows of each 32-row step
// stored in the slot order of the accumulator layout (hs2_bwd.h), so the
// A operand of the row contraction is one contiguous 8-element read.
#include "hs2_bwd.h"
#include "hs2_device.h"
#include "hs2_launch.h"

#include <algorithm>
#include <type_traits>

namespace hs2 {

namespace {

constexpr int MAX_ROWS = 64;

struct SparseBwdArgs {
  const void* q;        // [L, B, n_q, h_q, D] (this launch's layers)
  const void* o;
  const void* dout;
  const void* k;        // [B, n_kv, h_kv, D]
  const void* v;
  const int32_t* idx;   // [B, n_q, W]
  void* dq;             // [L, B, n_q, h_q, D]
  void* acc_k;          // [B, n_kv, h_kv, D]: fp32, or 64-bit fixed point
  void* acc_v;
  const float* acc_scale;   // fixed point: [0] = 2^F_K, [1] = 2^F_V
  int L, B, n_q, n_kv, h_q, h_kv, W;
  float scale, scale_log2;
};

// position of row rr (0..31 within its step) in the slot order
__device__ __forceinline__ int slot_pos(int rr) {
  const int hi = rr >> 4, x = rr & 15;
  return (x >> 2) * 8 + hi * 4 + (x & 3);
}

}  // namespace

template <typename T, int D, bool FIXED>
__global__ __launch_bounds__(512) void sparse_bwd_kernel(SparseBwdArgs a) {
  using Acc = std::conditional_t<FIXED, long long, float>;
  using OP = Op<T, D>;
  constexpr int DB = D / 16;                 // 16-wide head-dim blocks
  constexpr int DBW = DB / 2;                // per contraction wave
  constexpr int NSM = MAX_ROWS / 32;         // 32-row steps at most
  constexpr int TLD = MAX_ROWS + 16 / sizeof(T);   // padded: spreads the banks
  __shared__ __attribute__((aligned(16))) T s_p[2][32][TLD];
  __shared__ __attribute__((aligned(16))) T s_ds[2][32][TLD];
  __shared__ int s_key[2][32];               // buffer row of each tile key, -1 past the list
  __shared__ float s_m[4][8][16], s_l[4][8][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const int R = a.L * G;
  const int nrb = (R + 15) / 16;
  const int n_steps = (R + 31) / 32;

  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int g = wg % a.h_kv;
  const int bi = wg / a.h_kv;
  const int b = bi / a.n_q;
  const int i = bi - b * a.n_q;

  const T* kseq = reinterpret_cast<const T*>(a.k) + (size_t)b * a.n_kv * a.h_kv * D + g * D;
  const T* vseq = reinterpret_cast<const T*>(a.v) + (size_t)b * a.n_kv * a.h_kv * D + g * D;
  const size_t kstride = (size_t)a.h_kv * D;
  const int32_t* irow = a.idx + (size_t)bi * a.W;

  int n_valid = 0;
  for (int t = lane; t < a.W; t += 64) n_valid += (irow[t] >= 0) ? 1 : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n_valid += __shfl_xor(n_valid, m, 64);
  const int n_tiles = (n_valid + 31) / 32;

  // element offset of row r (layer r / G, head g * G + r % G) in the
  // [L, B, n_q, h_q, D] tensors
  auto row_off = [&](int r) {
    const int layer = r / G, hh = r - (r / G) * G;
    return ((((size_t)layer * a.B + b) * a.n_q + i) * a.h_q + g * G + hh) * D;
  };
  auto key_row = [&](int pos) -> size_t {
    return (size_t)irow[pos < n_valid ? pos : 0] * kstride;
  };

  for (int x = threadIdx.x; x < 2 * 32 * TLD; x += 512) {
    (&s_p[0][0][0])[x] = to_elem<T>(0.f);
    (&s_ds[0][0][0])[x] = to_elem<T>(0.f);
  }

  // ---- log-sum-exp of every row over the list, split over all 8 waves:
  // row block wave % nrb, tiles part, part + n_parts, ...
  {
    const int n_parts = 8 / nrb;
    const int rb = wave % nrb, part = wave / nrb;
    float m = -INFINITY, l = 0.f;
    if (part < n_parts) {
      Frag<T, D> qs;
      const int r = rb * 16 + l16;
      if (r < R) load_slice<T, D>(qs, reinterpret_cast<const T*>(a.q) + row_off(r), lane);
      else zero_slice<T, D>(qs);
      for (int t = part; t < n_tiles; t += n_parts) {
        const int base = t * 32;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          Frag<T, D> kf;
          load_slice<T, D>(kf, kseq + key_row(base + kb * 16 + l16), lane);
          const f32x4 s = dot_tile<T, D>(kf, qs, f32x4{0.f, 0.f, 0.f, 0.f});
          float x[4], tmax = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = base + kb * 16 + 4 * grp + e < n_valid ? s[e] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[e]);
          }
          const float m_new = fmaxf(m, tmax);
          if (m_new > -INFINITY) {
            float add = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) add += fast_exp2(x[e] - m_new);
            l = l * fast_exp2(m - m_new) + add;
            m = m_new;
          }
        }
      }
      // the four lane groups that share a row
#pragma unroll
      for (int mask = 16; mask <= 32; mask <<= 1) {
        const float mo = __shfl_xor(m, mask, 64);
        const float lo = __shfl_xor(l, mask, 64);
        const float mn = fmaxf(m, mo);
        if (mn > -INFINITY) {
          l = l * fast_exp2(m - mn) + lo * fast_exp2(mo - mn);
          m = mn;
        }
      }
      if (grp == 0) {
        s_m[rb][part][l16] = m;
        s_l[rb][part][l16] = l;
      }
    }
  }
  __syncthreads();

  // ---- row waves: Q, dO fragments, Delta, the combined log-sum-exp --------
  const bool row_wave = wave < nrb;
  const int my_row = wave * 16 + l16;
  const bool row_ok = row_wave && my_row < R;
  Frag<T, D> qf, df;
  float delta = 0.f, lse2 = INFINITY;             // INFINITY: P = 0 on padding rows
  if (row_ok) {
    const size_t off = row_off(my_row);
    load_slice<T, D>(qf, reinterpret_cast<const T*>(a.q) + off, lane);
    load_slice<T, D>(df, reinterpret_cast<const T*>(a.dout) + off, lane);
    Frag<T, D> of;
    load_slice<T, D>(of, reinterpret_cast<const T*>(a.o) + off, lane);
    const T* dp = reinterpret_cast<const T*>(&df.u[0]);
    const T* op = reinterpret_cast<const T*>(&of.u[0]);
#pragma unroll
    for (int e = 0; e < OP::SLICE; ++e) delta += to_f32(dp[e]) * to_f32(op[e]);
    float m = -INFINITY;
    for (int pt = 0; pt < 8 / nrb; ++pt) m = fmaxf(m, s_m[wave][pt][l16]);
    float l = 0.f;
    for (int pt = 0; pt < 8 / nrb; ++pt)
      if (s_m[wave][pt][l16] > -INFINITY) l += s_l[wave][pt][l16] * fast_exp2(s_m[wave][pt][l16] - m);
    if (l > 0.f) lse2 = m + __log2f(l);
  } else {
    zero_slice<T, D>(qf);
    zero_slice<T, D>(df);
  }
  delta += __shfl_xor(delta, 16, 64);
  delta += __shfl_xor(delta, 32, 64);

  // ---- contraction waves (4..7): constant B operands ------------------------
  // waves 4, 5: dK (B = Q rows); waves 6, 7: dV (B = dO rows); each takes
  // DBW of the DB head-dim blocks. Slot s of step st is row
  // 32 * st + slot_index(s, grp); the lane's column is d = 16 * dbk + l16.
  const bool contract_wave = wave >= 4;
  const int cw = wave - 4;
  const bool for_dk = cw < 2;
  const int dbk0 = (cw & 1) * DBW;
  T cu[DBW][NSM][8];
  if (contract_wave) {
    const T* src = reinterpret_cast<const T*>(for_dk ? a.q : a.dout);
#pragma unroll
    for (int bk = 0; bk < DBW; ++bk)
#pragma unroll
      for (int st = 0; st < NSM; ++st)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 32 * st + slot_index(s, grp);
          cu[bk][st][s] = (st < n_steps && r < R) ? src[row_off(r) + 16 * (dbk0 + bk) + l16]
                                                  : to_elem<T>(0.f);
        }
  }

  f32x4 dq[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) dq[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  Acc* accb = static_cast<Acc*>(for_dk ? a.acc_k : a.acc_v) + (size_t)b * a.n_kv * a.h_kv * D +
              (size_t)g * D;
  const float mul = for_dk ? a.scale : 1.f;
  double fix = 0.0;
  if constexpr (FIXED) fix = a.acc_scale[for_dk ? 0 : 1];

  // Software pipeline over the tiles: in step t the row waves work on tile t
  // (buffer t & 1) while the contraction waves contract tile t - 1 (the
  // other buffer) and issue its atomics. The row waves issue no atomics, so
  // their loads never wait behind them.
  for (int t = 0; t <= n_tiles; ++t) {
    if (row_wave && t < n_tiles) {
      const int base = t * 32;
      const int buf = t & 1;
      f32x4 p[2], ds[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const size_t kr = key_row(base + kb * 16 + l16);
        Frag<T, D> kf, vf;
        load_slice<T, D>(kf, kseq + kr, lane);
        load_slice<T, D>(vf, vseq + kr, lane);
        const f32x4 s = dot_tile<T, D>(kf, qf, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 dp = dot_tile<T, D>(vf, df, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = fast_exp2(s[e] * a.scale_log2 - lse2);
          if (base + kb * 16 + 4 * grp + e >= n_valid) x = 0.f;
          p[kb][e] = x;
          ds[kb][e] = x * (dp[e] - delta);
        }
      }
      // dQ^T += K_sel^T dS^T: K rows of this lane's 8 key slots
      TRows<T, D> tr;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const T* src = kseq + key_row(base + slot_index(s, grp)) + DB * l16;
        constexpr int BYTES = DB * sizeof(T);
        if constexpr (BYTES == 16) {
          *reinterpret_cast<uint4*>(&tr.raw[s][0]) = *reinterpret_cast<const uint4*>(src);
        } else if constexpr (BYTES == 8) {
          *reinterpret_cast<uint2*>(&tr.raw[s][0]) = *reinterpret_cast<const uint2*>(src);
        } else {
#pragma unroll
          for (int w = 0; w < BYTES / 16; ++w)
            reinterpret_cast<uint4*>(&tr.raw[s][0])[w] = reinterpret_cast<const uint4*>(src)[w];
        }
      }
      mma_t<T, D>(dq, tr, ds[0], ds[1]);
      // P^T and dS^T into LDS: key 16 kb + 4 grp + e, row my_row
      const int col = (my_row >> 5) * 32 + slot_pos(my_row & 31);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s_p[buf][kb * 16 + 4 * grp + e][col] = to_elem<T>(p[kb][e]);
          s_ds[buf][kb * 16 + 4 * grp + e][col] = to_elem<T>(ds[kb][e]);
        }
      if (wave == 0 && lane < 32) {
        const int pos = base + lane;
        s_key[buf][lane] = pos < n_valid ? irow[pos] : -1;
      }
    }
    if (contract_wave && t > 0) {
      // row contraction of tile t - 1: C[key 4 grp + e of kb][d = 16 dbk + l16]
      const int buf = (t - 1) & 1;
      const T(*tile)[TLD] = for_dk ? s_ds[buf] : s_p[buf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 c[DBW];
#pragma unroll
        for (int bk = 0; bk < DBW; ++bk) c[bk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NSM; ++st) {
          if (st >= n_steps) break;
          const T* arow = &tile[kb * 16 + l16][st * 32 + grp * 8];
          if constexpr (sizeof(T) == 2) {
            const bf16x8 au = *reinterpret_cast<const bf16x8*>(arow);
#pragma unroll
            for (int bk = 0; bk < DBW; ++bk) {
              bf16x8 bu;
#pragma unroll
              for (int s = 0; s < 8; ++s) bu[s] = cu[bk][st][s];
              c[bk] = OP::mma(au, bu, c[bk]);
            }
          } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const float av = arow[s];
#pragma unroll
              for (int bk = 0; bk < DBW; ++bk) c[bk] = OP::mma(av, cu[bk][st][s], c[bk]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = s_key[buf][kb * 16 + 4 * grp + e];
          if (key < 0) continue;
          Acc* dst = accb + (size_t)key * kstride + l16;
#pragma unroll
          for (int bk = 0; bk < DBW; ++bk) {
            if constexpr (FIXED) {
              const long long q = (long long)rint((double)(c[bk][e] * mul) * fix);
              atomicAdd(reinterpret_cast<unsigned long long*>(dst + 16 * (dbk0 + bk)),
                        (unsigned long long)q);
            } else {
              unsafeAtomicAdd(dst + 16 * (dbk0 + bk), c[bk][e] * mul);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if (row_ok) {
    T* dst = reinterpret_cast<T*>(a.dq) + row_off(my_row);
    store_t_row<T, D>(dst, dq, a.scale, AccIn{}, 0, grp);
  }
}

namespace {

template <typename T, int D>
hipError_t launch_sparse_bwd_t(const SparseBwdArgs& a, bool fixed, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.B * a.n_q * a.h_kv));
  if (fixed) hipLaunchKernelGGL((sparse_bwd_kernel<T, D, true>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((sparse_bwd_kernel<T, D, false>), grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_bwd(const SparseBwdPlan& p, hipStream_t st) {
  SparseBwdArgs a;
  a.q = p.q; a.o = p.o; a.dout = p.dout; a.k = p.k; a.v = p.v; a.idx = p.idx;
  a.dq = p.dq; a.acc_k = p.acc_k; a.acc_v = p.acc_v; a.acc_scale = p.acc_scale;
  if (p.fixed && !p.acc_scale) return hipErrorInvalidValue;
  a.L = p.layers; a.B = p.batch; a.n_q = p.n_q; a.n_kv = p.n_kv; a.h_q = p.h_q;
  a.h_kv = p.h_kv; a.W = p.width; a.scale = p.scale; a.scale_log2 = p.scale_log2;
  if (p.layers * (p.h_q / p.h_kv) > MAX_ROWS) return hipErrorInvalidValue;
  if (p.bf16) {
    if (p.head_dim == 128) return launch_sparse_bwd_t<__bf16, 128>(a, p.fixed, st);
    if (p.head_dim == 64) return launch_sparse_bwd_t<__bf16, 64>(a, p.fixed, st);
  } else {
    if (p.head_dim == 128) return launch_sparse_bwd_t<float, 128>(a, p.fixed, st);
    if (p.head_dim == 64) return launch_sparse_bwd_t<float, 64>(a, p.fixed, st);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// bounds for the fixed-point accumulators
// ---------------------------------------------------------------------------
namespace {

// Largest |Q| and |dO| entry and largest squared row norm of dO and of V.
// Sixteen lanes share a head-dim row (coalesced loads); non-negative floats
// order like their bit patterns, so integer atomicMax combines the waves.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_bound_kernel(const T* q, const T* dout, size_t q_rows,
                                                         const T* v, size_t v_rows, unsigned* mx) {
  constexpr int E = D / 16;                           // elements per lane of a row
  const int sub = threadIdx.x & 15;
  const size_t n = q_rows + v_rows;
  const size_t step = ((size_t)gridDim.x * blockDim.x) / 16;
  float mq = 0.f, mdo = 0.f, ndo = 0.f, nv = 0.f;
  for (size_t r = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 16; r < n; r += step) {
    float s = 0.f;
    if (r < q_rows) {
      const T* qr = q + r * D + sub * E;
      const T* dr = dout + r * D + sub * E;
#pragma unroll
      for (int x = 0; x < E; ++x) {
        const float b = to_f32(dr[x]);
        mq = fmaxf(mq, fabsf(to_f32(qr[x])));
        mdo = fmaxf(mdo, fabsf(b));
        s = fmaf(b, b, s);
      }
    } else {
      const T* vr = v + (r - q_rows) * D + sub * E;
#pragma unroll
      for (int x = 0; x < E; ++x) {
        const float b = to_f32(vr[x]);
        s = fmaf(b, b, s);
      }
    }
    // the row's sum of squares over its sixteen lanes (one row per group)
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (r < q_rows) ndo = fmaxf(ndo, s);
    else nv = fmaxf(nv, s);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mq = fmaxf(mq, __shfl_xor(mq, m, 64));
    mdo = fmaxf(mdo, __shfl_xor(mdo, m, 64));
    ndo = fmaxf(ndo, __shfl_xor(ndo, m, 64));
    nv = fmaxf(nv, __shfl_xor(nv, m, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&mx[0], __float_as_uint(mq));
    atomicMax(&mx[1], __float_as_uint(mdo));
    atomicMax(&mx[2], __float_as_uint(ndo));
    atomicMax(&mx[3], __float_as_uint(nv));
  }
}

// b = m 2^e with m < 1, so addends bounded by b, summed, stay below 2^61
// once scaled by 2^(61 - e); the rounding of each addend adds at most half a
// unit, far inside the two spare bits. Clamped so that 2^F and 2^-F stay
// finite in fp32 (an all-zero bound takes the finest scale).
__device__ int fixed_exponent(double b) {
  if (!(b > 0.0)) return 100;
  int e = 0;
  frexp(b, &e);
  return max(-64, min(100, 61 - e));
}

__global__ void bwd_scale_kernel(const unsigned* mx, float* scales, double rows, float softmax_scale) {
  const double mq = __uint_as_float(mx[0]), mdo = __uint_as_float(mx[1]);
  const double ndo = sqrt((double)__uint_as_float(mx[2])), nv = sqrt((double)__uint_as_float(mx[3]));
  // |dS| = P |dP - Delta| <= 2 P ||dO|| ||V||, and a key's P summed over all
  // rows of its KV head is at most the row count
  const int fk = fixed_exponent((double)softmax_scale * 2.0 * rows * ndo * nv * mq);
  const int fv = fixed_exponent(rows * mdo);
  scales[0] = ldexpf(1.f, fk);
  scales[1] = ldexpf(1.f, fv);
  scales[2] = ldexpf(1.f, -fk);
  scales[3] = ldexpf(1.f, -fv);
}

template <typename T, int D>
hipError_t launch_bounds_t(const SparseBwdBoundPlan& p, hipStream_t st) {
  const size_t n = p.q_rows + p.v_rows;
  const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>((n * 16 + 255) / 256, 4096));
  hipLaunchKernelGGL((bwd_bound_kernel<T, D>), dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<const T*>(p.q), reinterpret_cast<const T*>(p.dout), p.q_rows,
                     reinterpret_cast<const T*>(p.v), p.v_rows, p.maxima);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scale_kernel, dim3(1), dim3(1), 0, st, p.maxima, p.scales, p.rows, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_bwd_bounds(const SparseBwdBoundPlan& p, hipStream_t st) {
  if (p.bf16) {
    if (p.head_dim == 128) return launch_bounds_t<__bf16, 128>(p, st);
    if (p.head_dim == 64) return launch_bounds_t<__bf16, 64>(p, st);
  } else {
    if (p.head_dim == 128) return launch_bounds_t<float, 128>(p, st);
    if (p.head_dim == 64) return launch_bounds_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hs2
