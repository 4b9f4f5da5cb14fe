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
// indices in ascending order. One work-group (512 or 1024 threads, see
// token_threads) per query row.
// Rows of more than 128 * top_k candidates whose score pass also wrote the
// maxima of their 64-key segments take the segment path: the top_k-th
// largest maximum T bounds tau from below, so only the segments whose
// maximum reaches T (about top_k of them) are read, their keys >= T are
// gathered into LDS and the exact radix select runs there. Other long rows
// take a path that reads the row once: a threshold from 8192 sampled keys
// (2048 runs of 4, aimed at about 3k keys above the threshold), one pass
// gathering every key at or above it into LDS, and the exact radix select
// on that small set. Both fall back to the full passes when the gathered
// set is too small or does not fit; all paths select the same keys.
// Block mode with 64-token blocks takes its block maxima from the segment
// maxima as well.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

constexpr int SEL_THREADS = 1024;   // block mode, and the default of the shared helpers
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int LIST_CAP = 4096;       // top_k limit
constexpr int EQ_CAP = 2048;         // keys equal to the threshold sorted in LDS
constexpr int MAX_BLOCKS = 16384;    // block mode: candidate blocks per row
constexpr int MAX_TOP_BLOCKS = 256;

struct SelArgs {
  const float* scores; size_t stride;
  int32_t* idx;
  int flat0, n_q, n_kv, top_k, window, width;
  const int32_t* seq_len;            // keys per sequence (decode rows), or NULL
  int block_size, top_blocks;
  size_t seg_off;                    // 64-key segment maxima after each row, 0 = none
};

// Inclusive prefix sum over the NT threads of the block.
template <int NT = SEL_THREADS>
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
template <int NT = SEL_THREADS>
__device__ void find_digit(const int* hist, int nbins, int need, int* wsum, int* res) {
  const int per = nbins / NT > 0 ? nbins / NT : 1;
  const int t = threadIdx.x;
  const int rt = NT - 1 - t;                          // thread rt owns the high bins
  int v = 0;
  const int lo = rt * per;
  if (lo < nbins)
    for (int x = 0; x < per; ++x) v += hist[lo + x];
  const int incl = block_inclusive_scan<NT>(v, wsum); // bins above and including mine
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

template <int NT = SEL_THREADS>
__device__ void bitonic_sort(int* arr, int n_pow2) {
  for (int k = 2; k <= n_pow2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n_pow2; i += NT) {
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

// Keys of a full score row (index = position) ...
struct RowSrc {
  static constexpr bool kRow = true;
  const uint32_t* row;
  int n;
  __device__ __forceinline__ uint32_t key(int j) const { return row[j]; }
  __device__ __forceinline__ int index(int j) const { return j; }
};
// ... or of the candidates gathered into LDS (index stored beside the key).
struct CandSrc {
  static constexpr bool kRow = false;
  const uint32_t* keys;
  const int* idx;
  int n;
  __device__ __forceinline__ uint32_t key(int j) const { return keys[j]; }
  __device__ __forceinline__ int index(int j) const { return idx[j]; }
};

// Exact k-th largest key of src (12 + 12 + 8-bit radix passes with LDS
// histograms). Returns tau, how many keys == tau must be taken, and how many
// keys == tau exist.
template <int NT, class S>
__device__ void radix_kth(const S& src, int k, int* hist, int* wsum, int* res, uint32_t* tau,
                          int* need_eq, int* n_eq_total) {
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nbins = 1 << widths[pass];
    for (int x = threadIdx.x; x < nbins; x += NT) hist[x] = 0;
    __syncthreads();
    if constexpr (S::kRow) {
      // whole score rows: batched 16-byte loads
      constexpr int STRIDE = NT * 4;
      const int n_c = src.n;
      for (int jb = threadIdx.x * 4; jb < n_c; jb += 4 * STRIDE) {
        uint4 kv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kv[u] = *reinterpret_cast<const uint4*>(src.row + min(jb + u * STRIDE, (n_c - 1) & ~3));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = jb + u * STRIDE;
          const uint32_t ks[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < n_c && (ks[e] & pmask) == prefix)
              atomicAdd(&hist[(ks[e] >> sh) & (nbins - 1)], 1);
        }
      }
    } else {
      for (int j = threadIdx.x; j < src.n; j += NT) {
        const uint32_t kk = src.key(j);
        if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> sh) & (nbins - 1)], 1);
      }
    }
    __syncthreads();
    find_digit<NT>(hist, nbins, need, wsum, res);
    const int digit = res[0];
    need = res[1];
    if (pass == 2) *n_eq_total = hist[digit];
    prefix |= (uint32_t)digit << sh;
    pmask |= (uint32_t)(nbins - 1) << sh;
    __syncthreads();
  }
  *tau = prefix;
  *need_eq = need;
}

// Every key > tau into list, every key == tau into eqlist (when they fit).
// Whole score rows are read with batched 16-byte loads (rows are padded to
// a multiple of 256 floats, so a clamped quad never leaves the row).
template <int NT, class S>
__device__ void collect_above(const S& src, uint32_t tau, bool eq_fits, int* list, int* eqlist,
                              int* counters) {
  if (threadIdx.x < 2) counters[threadIdx.x] = 0;
  __syncthreads();
  if constexpr (S::kRow) {
    const int n_c = src.n;
    constexpr int STRIDE = NT * 4;
    for (int jb = threadIdx.x * 4; jb < n_c; jb += 4 * STRIDE) {
      uint4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kv[u] = *reinterpret_cast<const uint4*>(src.row + min(jb + u * STRIDE, (n_c - 1) & ~3));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * STRIDE;
        const uint32_t ks[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j + e >= n_c) continue;
          if (ks[e] > tau) list[atomicAdd(&counters[0], 1)] = j + e;
          else if (ks[e] == tau && eq_fits) eqlist[atomicAdd(&counters[1], 1)] = j + e;
        }
      }
    }
  } else {
    for (int j = threadIdx.x; j < src.n; j += NT) {
      const uint32_t kk = src.key(j);
      if (kk > tau) list[atomicAdd(&counters[0], 1)] = src.index(j);
      else if (kk == tau && eq_fits) eqlist[atomicAdd(&counters[1], 1)] = src.index(j);
    }
  }
  __syncthreads();
}

// Sort the tie list, append its need_eq lowest indices, sort the whole
// selection ascending and write it, followed by the window.
template <int NT>
__device__ void finish_selection(int* list, int* eqlist, int n_gt, int need_eq, int n_eq_total,
                                 bool eq_sorted_needed, int top_k, int32_t* out, int p,
                                 int window, int width) {
  if (eq_sorted_needed) {
    int n2 = 1;
    while (n2 < n_eq_total) n2 <<= 1;
    for (int x = n_eq_total + threadIdx.x; x < n2; x += NT) eqlist[x] = 0x7FFFFFFF;
    __syncthreads();
    if (n_eq_total > 1) bitonic_sort<NT>(eqlist, n2);
    for (int x = threadIdx.x; x < need_eq; x += NT) list[n_gt + x] = eqlist[x];
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < top_k) n2 <<= 1;
  for (int x = top_k + threadIdx.x; x < n2; x += NT) list[x] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort<NT>(list, n2);
  for (int t = threadIdx.x; t < top_k; t += NT) out[t] = list[t];
  write_window_and_pad(out, top_k, p, window, width);
}

constexpr int NSAMP = 8192;      // sampled keys per row (fast path)
constexpr int CAND_CAP = 4096;   // candidates gathered into LDS (fast path)

template <int NT>
__global__ __launch_bounds__(NT, 2048 / NT) void select_token_kernel(SelArgs a) {
  constexpr int NW = NT / 64;
  __shared__ int hist[4096];
  __shared__ int list[LIST_CAP];
  __shared__ int eqlist[EQ_CAP];
  __shared__ uint32_t ckey[CAND_CAP];
  __shared__ int cidx[CAND_CAP];
  __shared__ int wsum[NW];
  __shared__ int res[2];
  __shared__ int counters[2];

  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x;
  const int flat = a.flat0 + r;                       // b * n_q + i
  const int i = flat % a.n_q;
  const int p = (a.seq_len ? a.seq_len[flat / a.n_q] : a.n_kv) - a.n_q + i;
  const int n_c = max(0, p - a.window + 1);
  int32_t* out = a.idx + (size_t)flat * a.width;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(a.scores + (size_t)r * a.stride);

  if (n_c <= a.top_k) {
    for (int t = threadIdx.x; t < n_c; t += NT) out[t] = t;
    write_window_and_pad(out, n_c, p, a.window, a.width);
    return;
  }

  // ---- segment path: the row's 64-key segment maxima bound tau from below.
  // T = the top_k-th largest maximum: the top_k segments reaching it hold a
  // key >= T each, so tau >= T, and every key >= tau (ties included) lies in
  // a segment whose maximum is >= T. Gather the keys >= T of those segments
  // into LDS and select exactly there; only about top_k segments of the row
  // are read. Falls through when the segment list or the gathered keys do
  // not fit.
  if (a.seg_off && n_c >= 128 * a.top_k) {
    const int n_seg = (n_c + 63) >> 6;
    const uint32_t* srow = row + a.seg_off;
    uint32_t T;
    {
      int need_s, n_eq_s = 0;
      const RowSrc ms{srow, n_seg};
      radix_kth<NT>(ms, a.top_k, hist, wsum, res, &T, &need_s, &n_eq_s);
    }
    if (threadIdx.x == 0) counters[0] = 0;
    __syncthreads();
    // list[] <- ids of the segments whose maximum is >= T (in no set order)
    for (int sb = 0; sb < n_seg; sb += NT) {
      const int sg = sb + threadIdx.x;
      const bool f = sg < n_seg && srow[sg] >= T;
      const uint64_t m = __builtin_amdgcn_ballot_w64(f);
      if (m) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&counters[0], __popcll(m));
        base = __shfl(base, 0, 64);
        const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
        if (f && pos < LIST_CAP) list[pos] = sg;
      }
    }
    __syncthreads();
    const int n_list = counters[0];
    __syncthreads();
    if (n_list <= LIST_CAP) {
      if (threadIdx.x == 0) counters[0] = 0;
      __syncthreads();
      // 16 lanes per segment (one 16-byte quad each), four segments per
      // wave and four waves' worth of loads in flight per lane
      const int wave = threadIdx.x >> 6;
      constexpr int U = 4;
      for (int sb = wave * 4; sb < n_list; sb += NW * 4 * U) {
        uint4 kv[U];
        int j0[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = sb + u * NW * 4 + (lane >> 4);
          const int sg = list[min(t, n_list - 1)];
          j0[u] = t < n_list ? sg * 64 + (lane & 15) * 4 : n_c;
          kv[u] = *reinterpret_cast<const uint4*>(row + sg * 64 + (lane & 15) * 4);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t ks[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool f = (j0[u] + e < n_c) && ks[e] >= T;
            const uint64_t m = __builtin_amdgcn_ballot_w64(f);
            if (m) {
              int base = 0;
              if (lane == 0) base = atomicAdd(&counters[0], __popcll(m));
              base = __shfl(base, 0, 64);
              const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
              if (f && pos < CAND_CAP) {
                ckey[pos] = ks[e];
                cidx[pos] = j0[u] + e;
              }
            }
          }
        }
      }
      __syncthreads();
      const int n_cand = counters[0];
      __syncthreads();
      if (n_cand <= CAND_CAP) {
        const CandSrc cs{ckey, cidx, n_cand};
        uint32_t tau;
        int need_eq, n_eq_total = 0;
        radix_kth<NT>(cs, a.top_k, hist, wsum, res, &tau, &need_eq, &n_eq_total);
        if (n_eq_total <= EQ_CAP) {
          collect_above<NT>(cs, tau, true, list, eqlist, counters);
          finish_selection<NT>(list, eqlist, a.top_k - need_eq, need_eq, n_eq_total, true,
                               a.top_k, out, p, a.window, a.width);
          return;
        }
      }
    }
    __syncthreads();
  }

  // ---- fast path: a conservative threshold from a strided sample, one pass
  // that gathers every key at or above it into LDS, exact selection there.
  // Exact whenever at least top_k keys were gathered (then the top_k-th
  // largest key, and every key equal to it, is among them).
  if (n_c >= 4 * a.top_k && n_c >= 16384) {
    for (int x = threadIdx.x; x < 4096; x += NT) hist[x] = 0;
    if (threadIdx.x == 0) counters[0] = 0;
    __syncthreads();
    // 8192 sampled keys: 2048 runs of 4 spread over the row (short runs keep
    // clustered structure from skewing the sample); two histogram levels
    // place the threshold at 24-bit precision
    constexpr int RPT = 2048 / NT;                    // runs per thread
    constexpr int SK = 4 * RPT;
    uint32_t sk[SK];
    // (re)read this thread's sampled keys: they are not kept in registers
    // across the gather pass, a retry reads them again
    auto load_sample = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int run = RPT * threadIdx.x + q;
        const int sj = (int)(((long long)run * (n_c - 4)) / 2047) / 4 * 4;
        const uint4 sv = *reinterpret_cast<const uint4*>(row + sj);
        sk[4 * q] = sv.x; sk[4 * q + 1] = sv.y; sk[4 * q + 2] = sv.z; sk[4 * q + 3] = sv.w;
      }
    };
    load_sample();
#pragma unroll
    for (int e = 0; e < SK; ++e) atomicAdd(&hist[sk[e] >> 20], 1);
    __syncthreads();
    // up to two attempts: a gather that overflows retries with a higher
    // threshold, one that catches fewer than top_k keys with a lower one
    int rank = min(NSAMP, max(8, (int)(((long long)3 * a.top_k * NSAMP + n_c - 1) / n_c)));
    int n_cand = 0;
    for (int attempt = 0; attempt < 2; ++attempt) {
    if (attempt > 0) {
      if (n_cand > CAND_CAP) rank = max(1, rank * 3 / 5);
      else rank = min(NSAMP, rank * 2);
      for (int x = threadIdx.x; x < 4096; x += NT) hist[x] = 0;
      if (threadIdx.x == 0) counters[0] = 0;
      __syncthreads();
      load_sample();
#pragma unroll
      for (int e = 0; e < SK; ++e) atomicAdd(&hist[sk[e] >> 20], 1);
      __syncthreads();
    }
    find_digit<NT>(hist, 4096, rank, wsum, res);
    const uint32_t top12 = (uint32_t)res[0];
    const int rank2 = res[1];
    __syncthreads();
    for (int x = threadIdx.x; x < 4096; x += NT) hist[x] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < SK; ++e)
      if ((sk[e] >> 20) == top12) atomicAdd(&hist[(sk[e] >> 8) & 4095], 1);
    __syncthreads();
    find_digit<NT>(hist, 4096, rank2, wsum, res);
    const uint32_t v_s = (top12 << 20) | ((uint32_t)res[0] << 8);
    // eight 16-byte loads in flight per thread
    constexpr int STRIDE = NT * 4;
    for (int jb = threadIdx.x * 4; jb < n_c; jb += 8 * STRIDE) {
      // branch-free loads so all eight stay in flight: a position past the
      // row is clamped to its last aligned quad and masked below (rows are
      // padded to a multiple of 256 floats, so a quad never leaves them)
      uint4 kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j0 = min(jb + u * STRIDE, (n_c - 1) & ~3);
        kv[u] = *reinterpret_cast<const uint4*>(row + j0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j0 = jb + u * STRIDE;
        const uint32_t ks[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool f = (j0 + e < n_c) && ks[e] >= v_s;
          const uint64_t m = __builtin_amdgcn_ballot_w64(f);
          if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&counters[0], __popcll(m));
            base = __shfl(base, 0, 64);
            const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
            if (f && pos < CAND_CAP) {
              ckey[pos] = ks[e];
              cidx[pos] = j0 + e;
            }
          }
        }
      }
    }
    __syncthreads();
    n_cand = counters[0];
    __syncthreads();
    if (n_cand >= a.top_k && n_cand <= CAND_CAP) break;
    }
    if (n_cand >= a.top_k && n_cand <= CAND_CAP) {
      const CandSrc cs{ckey, cidx, n_cand};
      uint32_t tau;
      int need_eq, n_eq_total = 0;
      radix_kth<NT>(cs, a.top_k, hist, wsum, res, &tau, &need_eq, &n_eq_total);
      if (n_eq_total <= EQ_CAP) {
        collect_above<NT>(cs, tau, true, list, eqlist, counters);
        finish_selection<NT>(list, eqlist, a.top_k - need_eq, need_eq, n_eq_total, true, a.top_k,
                             out, p, a.window, a.width);
        return;
      }
    }
    __syncthreads();
  }

  // ---- general path: radix passes over the whole row ----
  const RowSrc rs{row, n_c};
  uint32_t tau;
  int need_eq, n_eq_total = 0;
  radix_kth<NT>(rs, a.top_k, hist, wsum, res, &tau, &need_eq, &n_eq_total);
  const int n_gt = a.top_k - need_eq;
  const bool eq_fits = n_eq_total <= EQ_CAP;
  collect_above<NT>(rs, tau, eq_fits, list, eqlist, counters);
  if (!eq_fits) {
    // many exact ties: walk the row in index order and keep the first need_eq
    int taken = 0;
    for (int base = 0; base < n_c && taken < need_eq; base += NT) {
      const int j = base + threadIdx.x;
      const int f = (j < n_c && row[j] == tau) ? 1 : 0;
      const int incl = block_inclusive_scan<NT>(f, wsum);
      if (f && taken + incl - 1 < need_eq) list[n_gt + taken + incl - 1] = j;
      if (threadIdx.x == NT - 1) res[0] = incl;
      __syncthreads();
      taken += res[0];
      __syncthreads();
    }
  }
  finish_selection<NT>(list, eqlist, n_gt, need_eq, n_eq_total, eq_fits, a.top_k, out, p,
                       a.window, a.width);
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
  const int p = (a.seq_len ? a.seq_len[flat / a.n_q] : a.n_kv) - a.n_q + i;
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

  // block maxima (as order-preserving keys + 1, so 0 can mean "taken"); for
  // 64-token blocks the score pass already wrote them after the row
  if (a.seg_off && bs == 64) {
    const uint32_t* srow = row + a.seg_off;
    for (int beta = threadIdx.x; beta < n_blocks; beta += SEL_THREADS) bkey[beta] = srow[beta] + 1u;
  } else
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

// Work-group size of a token-select launch. Two 512-thread work-groups fit
// a CU (one 1024-thread one does), so one row's serial steps (threshold,
// radix passes over the gathered keys, sorts) overlap another row's read;
// that measured faster for launches of many rows of moderate length (32K
// prefill 3.5 -> 2.3 ms, 8K chunk on 262K 2.5 -> 2.2 ms), and for rows that
// take the segment path, which read only about top_k segments (16K chunk on
// 1M 3.5 -> 2.95 ms). Other rows of a million candidates (24.4 vs 21.3 ms
// when they read the whole row) and launches of few rows (decode) keep 1024
// threads per row.
int token_threads(const SelectPlan& p) {
  const long long longest = (long long)p.n_kv - p.window;
  if (p.rows < 512) return 1024;
  if (p.seg_off && !p.block_mode && longest >= 128LL * p.top_k) return 512;
  return longest < (1 << 19) ? 512 : 1024;
}

hipError_t launch_select(const SelectPlan& p, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  SelArgs a;
  a.scores = p.scores; a.stride = p.score_stride; a.idx = p.idx;
  a.flat0 = p.flat0; a.n_q = p.n_q; a.n_kv = p.n_kv; a.seq_len = p.seq_len;
  a.top_k = p.top_k; a.window = p.window; a.width = p.width;
  a.block_size = p.block_size; a.top_blocks = p.top_blocks;
  a.seg_off = p.seg_off;
  if (p.block_mode)
    hipLaunchKernelGGL(select_block_kernel, dim3(p.rows), dim3(SEL_THREADS), 0, st, a);
  else if (token_threads(p) == 512)
    hipLaunchKernelGGL(select_token_kernel<512>, dim3(p.rows), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(select_token_kernel<1024>, dim3(p.rows), dim3(1024), 0, st, a);
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
