// One decode step over a growing KV cache: each sequence appends its new
// token's K and V rows to the cache, which the full layer and every sparse
// layer of the block then read (HySparse2 pages: hitechexpert.top, section
// "Two-Level KV Sharing": one KV cache serves the full layer and the sparse
// layers that reuse it; blog.lynxflow.co, section "Token-Level Sparse
// Selection and Deployment Optimization": decode is bound by memory
// bandwidth, so the cache is read in place and never copied).
//
// Chunked prefill over a paged pool appends a chunk of rows per sequence
// (kv_stage_kernel): the new rows go into their pages, and the sequences
// with two or more new tokens get a contiguous staging copy of all their
// rows, which the prefill kernels then read.
//
// The per-sequence lengths reach the GPU as kernel arguments (copied at
// launch, so the call stays asynchronous and keeps no host buffer alive)
// and land in a small device array that the decode kernels read.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

namespace {

constexpr int LENS_PER_LAUNCH = 256;

struct LensArg {
  int32_t v[LENS_PER_LAUNCH];
};

}  // namespace

// seq_len[first + i] = lens[i] + 1: the keys held once the new row is in
__global__ __launch_bounds__(LENS_PER_LAUNCH) void set_lens_kernel(LensArg lens, int first,
                                                                   int count, int32_t* seq_len) {
  const int i = threadIdx.x;
  if (i < count) seq_len[first + i] = lens.v[i] + 1;
}

// one work-group per (sequence, K or V); the row of every KV head is
// contiguous (h_kv * head_dim elements), copied as 16-byte chunks
__global__ __launch_bounds__(256) void kv_append_kernel(const char* k_new, const char* v_new,
                                                        char* k_cache, char* v_cache,
                                                        const int32_t* seq_len, KvRows kv,
                                                        int row_bytes) {
  const int b = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const char* src = (is_v ? v_new : k_new) + (size_t)b * row_bytes;
  char* dst = (is_v ? v_cache : k_cache) + kv.row(b, seq_len[b] - 1) * row_bytes;
  for (int c = threadIdx.x; c < row_bytes / 16; c += blockDim.x)
    reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
}

// Chunked prefill: every position a work-group visits is one K row and one
// V row of row_bytes, moved as 16-byte chunks; consecutive threads take
// consecutive chunks of a row, so each row is one coalesced run
__global__ __launch_bounds__(256) void kv_stage_kernel(StageSeqs s, const char* k_new,
                                                       const char* v_new, char* k_pool,
                                                       char* v_pool, char* k_stage, char* v_stage,
                                                       KvRows kv, int row_bytes) {
  const int g = blockIdx.x;
  int i = 0;
  while (i + 1 < s.n && g >= s.blk0[i + 1]) ++i;
  const int j_first = s.r0[i] + (g - s.blk0[i]) * STAGE_ROWS;
  const int j_end = min(j_first + STAGE_ROWS, s.end[i]);
  const int chunks = row_bytes >> 4;
  const int lens = s.lens[i];
  const long long st0 = s.st0[i];
  const int32_t* table = kv.table + (size_t)s.b[i] * kv.max_pages;
  for (int e = threadIdx.x; e < (j_end - j_first) * chunks; e += blockDim.x) {
    const int jr = e / chunks;
    const int c = e - jr * chunks;
    const int j = j_first + jr;
    const size_t prow = kv.page_row(table[j >> kv.page_shift], j);
    uint4* kp = reinterpret_cast<uint4*>(k_pool + prow * row_bytes) + c;
    uint4* vp = reinterpret_cast<uint4*>(v_pool + prow * row_bytes) + c;
    uint4 kx, vx;
    if (j >= lens) {
      const size_t nrow = (size_t)(s.q0[i] + j - lens);
      kx = reinterpret_cast<const uint4*>(k_new + nrow * row_bytes)[c];
      vx = reinterpret_cast<const uint4*>(v_new + nrow * row_bytes)[c];
      *kp = kx;
      *vp = vx;
    } else {
      kx = *kp;
      vx = *vp;
    }
    if (st0 >= 0) {
      const size_t srow = (size_t)(st0 + j);
      reinterpret_cast<uint4*>(k_stage + srow * row_bytes)[c] = kx;
      reinterpret_cast<uint4*>(v_stage + srow * row_bytes)[c] = vx;
    }
  }
}

hipError_t launch_kv_stage(const StageSeqs& s, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, void* k_stage, void* v_stage, const KvRows& kv,
                           int row_bytes, hipStream_t st) {
  if (s.n <= 0 || s.blk0[s.n] <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_stage_kernel, dim3((unsigned)s.blk0[s.n]), dim3(256), 0, st, s,
                     reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                     reinterpret_cast<char*>(k_pool), reinterpret_cast<char*>(v_pool),
                     reinterpret_cast<char*>(k_stage), reinterpret_cast<char*>(v_stage), kv,
                     row_bytes);
  return hipGetLastError();
}

hipError_t launch_set_lens(const int32_t* lens_host, int first, int count, int32_t* seq_len,
                           hipStream_t st) {
  for (int i0 = 0; i0 < count; i0 += LENS_PER_LAUNCH) {
    LensArg arg;
    const int n = count - i0 < LENS_PER_LAUNCH ? count - i0 : LENS_PER_LAUNCH;
    for (int i = 0; i < n; ++i) arg.v[i] = lens_host[i0 + i];
    hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(LENS_PER_LAUNCH), 0, st, arg, first + i0, n,
                       seq_len);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* seq_len, int batch, const KvRows& kv, int row_bytes,
                            hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)batch * 2), dim3(256), 0, st,
                     reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                     reinterpret_cast<char*>(k_cache), reinterpret_cast<char*>(v_cache), seq_len,
                     kv, row_bytes);
  return hipGetLastError();
}

}  // namespace hs2
