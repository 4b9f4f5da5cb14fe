// Selection: which keys each sparse layer will read.
//
// Token mode (HySparse2 pages: "Xiaomi Unveils HySparse2", section
// "Token-Level Selection and Unified Local Access"; bibibi.cc, section
// "Article"): the most recent `window` tokens are always kept, and the
// `top_k` best candidates j <= p - window are taken by (-S, j), i.e. ties go
// to the lower index. Block mode (the previous generation's 64-token groups,
// bibibi.cc, section "Article") ranks candidate blocks by their max score.
//
// Token top-k is an exact radix select on the fp32 bit pattern of S (S >= 0,
// so the bits order like the values): three histogram passes (12 + 12 + 8
// bits) fix the k-th largest key tau, one pass collects every key > tau and
// the lowest-index keys == tau, and a bitonic sort in LDS puts the chosen
// indices in ascending order. One 1024-thread work-group per query row.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int LIST_CAP = 4096;       // top_k limit and tie-list capacity
constexpr int MAX_BLOCKS = 16384;    // block mode: candidate blocks per row
constexpr int MAX_TOP_BLOCKS = 256;

struct SelArgs {
  const float* scores; size_t stride;
  int32_t* idx;
  int flat0, n_q, n_kv, top_k, window, width;
  int block_size, top_blocks;
};

// Inclusive prefix sum over the 1024 threads of the block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  __syncthreads();
  return v + off;
}

__device__ __forceinline__ void write_window_and_pad(int32_t* out, int n_sel, int p, int window,
                                                     int width) {
  const int w0 = max(0, p - window + 1);
  const int nw = p - w0 + 1;
  for (int t = threadIdx.x; t < width - n_sel; t += blockDim.x)
    out[n_sel + t] = (t < nw) ? (w0 + t) : -1;
}

// Find the digit holding the `need`-th largest key among hist[0..nbins) and
// return (digit, how many of the needed keys are still inside that digit).
__device__ void find_digit(const int* hist, int nbins, int need, int* wsum, int* res) {
  const int per = nbins / SEL_THREADS > 0 ? nbins / SEL_THREADS : 1;
  const int t = threadIdx.x;
  const int rt = SEL_THREADS - 1 - t;                 // thread rt owns the high bins
  int v = 0;
  const int lo = rt * per;
  if (lo < nbins)
    for (int x = 0; x < per; ++x) v += hist[lo + x];
  const int incl = block_inclusive_scan(v, wsum);     // bins above and including mine
  const int above = incl - v;
  if (lo < nbins && above < need && need <= incl) {
    int acc = above;
    for (int x = per - 1; x >= 0; --x) {
      const int c = hist[lo + x];
      if (acc + c >= need) {
        res[0] = lo + x;
        res[1] = need - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__device__ void bitonic_sort(int* arr, int n_pow2) {
  for (int k = 2; k <= n_pow2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n_pow2; i += SEL_THREADS) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool asc = (i & k) == 0;
          const int x = arr[i], y = arr[ixj];
          if ((x > y) == asc) {
            arr[i] = y;
            arr[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
}

__global__ __launch_bounds__(SEL_THREADS) void select_token_kernel(SelArgs a) {
  __shared__ int hist[4096];
  __shared__ int list[LIST_CAP];
  __shared__ int eqlist[LIST_CAP];
  __shared__ int wsum[SEL_WAVES];
  __shared__ int res[2];
  __shared__ int counters[2];

  const int r = blockIdx.x;
  const int flat = a.flat0 + r;                       // b * n_q + i
  const int i = flat % a.n_q;
  const int p = a.n_kv - a.n_q + i;
  const int n_c = max(0, p - a.window + 1);
  int32_t* out = a.idx + (size_t)flat * a.width;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(a.scores + (size_t)r * a.stride);

  if (n_c <= a.top_k) {
    for (int t = threadIdx.x; t < n_c; t += SEL_THREADS) out[t] = t;
    write_window_and_pad(out, n_c, p, a.window, a.width);
    return;
  }

  // ---- radix select of the top_k-th largest key ----
  uint32_t prefix = 0, pmask = 0;
  int need = a.top_k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  int n_eq_total = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = widths[pass];
    const int nbins = 1 << nb;
    for (int x = threadIdx.x; x < nbins; x += SEL_THREADS) hist[x] = 0;
    __syncthreads();
    for (int j = threadIdx.x * 4; j < n_c; j += SEL_THREADS * 4) {
      uint4 kv;
      if (j + 3 < n_c) {
        kv = *reinterpret_cast<const uint4*>(row + j);
      } else {
        kv.x = row[j];
        kv.y = (j + 1 < n_c) ? row[j + 1] : 0xFFFFFFFFu;
        kv.z = (j + 2 < n_c) ? row[j + 2] : 0xFFFFFFFFu;
        kv.w = 0xFFFFFFFFu;
      }
      const uint32_t ks[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (j + e < n_c && (ks[e] & pmask) == prefix)
          atomicAdd(&hist[(ks[e] >> sh) & (nbins - 1)], 1);
      }
    }
    __syncthreads();
    find_digit(hist, nbins, need, wsum, res);
    const int digit = res[0];
    need = res[1];
    if (pass == 2) n_eq_total = hist[digit];
    prefix |= (uint32_t)digit << sh;
    pmask |= (uint32_t)(nbins - 1) << sh;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const int need_eq = need;                       // keys == tau to take
  const int n_gt = a.top_k - need_eq;

  // ---- collect keys > tau and (if they fit) every key == tau ----
  if (threadIdx.x < 2) counters[threadIdx.x] = 0;
  __syncthreads();
  const bool eq_fits = n_eq_total <= LIST_CAP;
  for (int j = threadIdx.x; j < n_c; j += SEL_THREADS) {
    const uint32_t key = row[j];
    if (key > tau) {
      list[atomicAdd(&counters[0], 1)] = j;
    } else if (key == tau && eq_fits) {
      eqlist[atomicAdd(&counters[1], 1)] = j;
    }
  }
  __syncthreads();

  if (eq_fits) {
    int n2 = 1;
    while (n2 < n_eq_total) n2 <<= 1;
    for (int x = n_eq_total + threadIdx.x; x < n2; x += SEL_THREADS) eqlist[x] = 0x7FFFFFFF;
    __syncthreads();
    if (n_eq_total > 1) bitonic_sort(eqlist, n2);
    for (int x = threadIdx.x; x < need_eq; x += SEL_THREADS) list[n_gt + x] = eqlist[x];
  } else {
    // many exact ties: walk the row in index order and keep the first need_eq
    int taken = 0;
    for (int base = 0; base < n_c && taken < need_eq; base += SEL_THREADS) {
      const int j = base + threadIdx.x;
      const int f = (j < n_c && row[j] == tau) ? 1 : 0;
      const int incl = block_inclusive_scan(f, wsum);
      if (f && taken + incl - 1 < need_eq) list[n_gt + taken + incl - 1] = j;
      if (threadIdx.x == SEL_THREADS - 1) res[0] = incl;
      __syncthreads();
      taken += res[0];
      __syncthreads();
    }
  }
  __syncthreads();

  int n2 = 1;
  while (n2 < a.top_k) n2 <<= 1;
  for (int x = a.top_k + threadIdx.x; x < n2; x += SEL_THREADS) list[x] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort(list, n2);
  for (int t = threadIdx.x; t < a.top_k; t += SEL_THREADS) out[t] = list[t];
  write_window_and_pad(out, a.top_k, p, a.window, a.width);
}

// ---------------------------------------------------------------------------
// block mode
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long max_u64(unsigned long long x, unsigned long long y) {
  return x > y ? x : y;
}

__global__ __launch_bounds__(SEL_THREADS) void select_block_kernel(SelArgs a) {
  __shared__ uint32_t bkey[MAX_BLOCKS];
  __shared__ unsigned long long wbest[SEL_WAVES];
  __shared__ int chosen[MAX_TOP_BLOCKS];
  __shared__ int sorted_blocks[MAX_TOP_BLOCKS];
  __shared__ int offs[MAX_TOP_BLOCKS + 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x;
  const int flat = a.flat0 + r;                       // b * n_q + i
  const int i = flat % a.n_q;
  const int p = a.n_kv - a.n_q + i;
  const int n_c = max(0, p - a.window + 1);
  const int bs = a.block_size;
  const int n_blocks = (n_c + bs - 1) / bs;
  int32_t* out = a.idx + (size_t)flat * a.width;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(a.scores + (size_t)r * a.stride);

  if (n_blocks <= a.top_blocks) {
    for (int t = threadIdx.x; t < n_c; t += SEL_THREADS) out[t] = t;
    write_window_and_pad(out, n_c, p, a.window, a.width);
    return;
  }

  // block maxima (as order-preserving keys + 1, so 0 can mean "taken")
  for (int beta = wave; beta < n_blocks; beta += SEL_WAVES) {
    const int lo = beta * bs, hi = min(n_c, lo + bs);
    uint32_t m = 0;
    for (int j = lo + lane; j < hi; j += 64) m = max(m, row[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if (lane == 0) bkey[beta] = m + 1u;
  }
  __syncthreads();

  for (int t = 0; t < a.top_blocks; ++t) {
    unsigned long long best = 0;
    for (int beta = threadIdx.x; beta < n_blocks; beta += SEL_THREADS) {
      const unsigned long long c =
          ((unsigned long long)bkey[beta] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)beta);
      best = max_u64(best, c);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) best = max_u64(best, (unsigned long long)__shfl_xor((long long)best, o, 64));
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long bb = 0;
      for (int w = 0; w < SEL_WAVES; ++w) bb = max_u64(bb, wbest[w]);
      const int beta = (int)(0xFFFFFFFFu - (uint32_t)(bb & 0xFFFFFFFFull));
      chosen[t] = beta;
      bkey[beta] = 0u;
    }
    __syncthreads();
  }

  // ascending block order, then expand to candidate tokens
  if (threadIdx.x < a.top_blocks) {
    const int c = chosen[threadIdx.x];
    int rank = 0;
    for (int u = 0; u < a.top_blocks; ++u) rank += (chosen[u] < c) ? 1 : 0;
    sorted_blocks[rank] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int u = 0; u < a.top_blocks; ++u) {
      offs[u] = acc;
      const int lo = sorted_blocks[u] * bs;
      acc += min(n_c, lo + bs) - lo;
    }
    offs[a.top_blocks] = acc;
  }
  __syncthreads();
  for (int u = 0; u < a.top_blocks; ++u) {
    const int lo = sorted_blocks[u] * bs;
    const int cnt = offs[u + 1] - offs[u];
    for (int t = threadIdx.x; t < cnt; t += SEL_THREADS) out[offs[u] + t] = lo + t;
  }
  const int n_sel = offs[a.top_blocks];
  write_window_and_pad(out, n_sel, p, a.window, a.width);
}

hipError_t launch_select(const SelectPlan& p, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  SelArgs a;
  a.scores = p.scores; a.stride = p.score_stride; a.idx = p.idx;
  a.flat0 = p.flat0; a.n_q = p.n_q; a.n_kv = p.n_kv;
  a.top_k = p.top_k; a.window = p.window; a.width = p.width;
  a.block_size = p.block_size; a.top_blocks = p.top_blocks;
  if (p.block_mode)
    hipLaunchKernelGGL(select_block_kernel, dim3(p.rows), dim3(SEL_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(select_token_kernel, dim3(p.rows), dim3(SEL_THREADS), 0, st, a);
  return hipGetLastError();
}

__global__ void export_scores_kernel(const float* src, int n_cand, int n_kv, float* dst) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n_kv) dst[j] = (j < n_cand) ? src[j] : -1.f;
}

hipError_t launch_export_scores(const float* src, int n_cand, int n_kv, float* dst,
                                hipStream_t st) {
  hipLaunchKernelGGL(export_scores_kernel, dim3((n_kv + 255) / 256), dim3(256), 0, st, src,
                     n_cand, n_kv, dst);
  return hipGetLastError();
}

}  // namespace hs2
