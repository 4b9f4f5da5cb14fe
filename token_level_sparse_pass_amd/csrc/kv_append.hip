// One decode step over a growing KV cache: each sequence appends its new
// token's K and V rows to the cache, which the full layer and every sparse
// layer of the block then read (HySparse2 pages: hitechexpert.top, section
// "Two-Level KV Sharing": one KV cache serves the full layer and the sparse
// layers that reuse it; blog.lynxflow.co, section "Token-Level Sparse
// Selection and Deployment Optimization": decode is bound by memory
// bandwidth, so the cache is read in place and never copied).
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
