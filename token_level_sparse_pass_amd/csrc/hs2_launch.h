// Host-side launch descriptions of the Hybrid Block kernels. Each launcher
// checks nothing: the C ABI layer validates every argument first.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace hs2 {

// Raise a kernel's dynamic-LDS limit to `bytes` once per device (the
// attribute is per device; the flag is set only after the call succeeded).
// Kernels with one cache slot each, so `Tag` distinguishes the callers.
template <typename Tag>
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Where key j of sequence b lives in a K/V buffer of [rows][h_kv][d]: a
// contiguous cache holds each sequence's n_kv rows back to back; a paged
// pool maps j through the sequence's page-table row (2^page_shift rows per
// page). Page ids are clamped to the pool, so a bad id reads a wrong page
// but never leaves the buffer.
struct KvRows {
  const int32_t* table = nullptr;   // [batch][max_pages], or NULL
  int n_kv = 0;
  int page_shift = 0, max_pages = 0, n_pages = 0;
  __device__ __forceinline__ bool paged() const { return table != nullptr; }
  __device__ __forceinline__ size_t page_row(int page_id, int j) const {
    const int pid = min(max(page_id, 0), n_pages - 1);
    return ((size_t)pid << page_shift) + (j & ((1 << page_shift) - 1));
  }
  __device__ __forceinline__ size_t row(int b, int j) const {
    if (!table) return (size_t)b * n_kv + j;
    return page_row(table[(size_t)b * max_pages + (j >> page_shift)], j);
  }
};


// Shape shared by the full-layer kernels.
struct Shape {
  int batch, n_q, n_kv, h_q, h_kv, head_dim;
  bool bf16;
  float scale_log2;       // softmax scale * log2(e)
};

// A launch over packed sequences of different lengths (bf16 / head_dim 128
// prefill): sequence s has nq[s] queries from token q0[s] and nkv[s] keys
// from token kv0[s] of the packed tensors, its transposed V starts vt0[s]
// 64-key tiles (all KV heads counted) into the workspace copy, and its
// row tiles are work-group rows tile0[s] .. tile0[s+1] (times h_kv).
constexpr int VARLEN_MAX_SEQS = 32;
struct VarlenSeqs {
  int n = 0;
  int tile0[VARLEN_MAX_SEQS + 1];
  int q0[VARLEN_MAX_SEQS], kv0[VARLEN_MAX_SEQS];
  int nq[VARLEN_MAX_SEQS], nkv[VARLEN_MAX_SEQS];
  int vt0[VARLEN_MAX_SEQS];
};
// rows (query, head-of-group pairs) per work-group of the bf16 prefill kernel
int prefill_rows_per_tile();

// Pass 1 (full causal attention) for prefill-shaped calls.
// stats: [3][batch][h_q][n_q] floats: m2 (row max in log2 units), l (row sum
// of 2^(t - m2)) and 1/l; lse (nullable): natural-log LSE.
// vt (bf16, head_dim 128 only): workspace for V transposed to
// [batch][h_kv][head_dim][vt_keys] (keys >= n_kv zero-filled), which lets
// the PV product read V with 16-byte LDS loads; NULL selects the generic
// kernel.
struct FwdPlan {
  Shape s;
  const void* q; const void* k; const void* v;
  void* o;
  float* stats;
  float* lse;
  void* vt; int vt_keys;
  // non-NULL (bf16 / head_dim 128 only): packed sequences; s.batch, s.n_q,
  // s.n_kv are then unused, stats / lse hold one block per sequence (stats:
  // 3 planes of h_q x nq at 3 * h_q * q0; lse: h_q x nq at h_q * q0), and
  // vt must already hold every sequence's transposed V
  const VarlenSeqs* vl = nullptr;
};
bool prefill_uses_vt(const Shape& s);
int vt_keys_for(int n_kv);
// Fills vt from v (a no-op unless the bf16 kernel is used); must run before
// launch_attn_fwd_prefill on the same stream.
hipError_t launch_v_transpose(const FwdPlan& p, hipStream_t st);
hipError_t launch_attn_fwd_prefill(const FwdPlan& p, hipStream_t st);

// Decode (n_q == 1): split-KV pass 1 that also stores every raw logit (q.k)
// so the score needs no second read of K; partials are merged by
// the combine step. part: [batch][h_q][n_split][head_dim + 2] floats,
// logits: [batch][h_q][logits_stride] floats (one row of raw logits q.k per
// sequence and query head), with logits_stride a multiple of 64 that is
// >= n_kv, so whole tiles of a ragged last split stay inside.
struct DecodePlan {
  Shape s;
  const void* q; const void* k; const void* v;
  void* o;
  float* stats;
  float* lse;
  float* part;
  float* logits; size_t logits_stride;
  int keys_per_split;     // multiple of 64
  int n_split;
  // optional [batch] device array: sequence b holds seq_len[b] <= n_kv keys
  // (its query sits at seq_len[b] - 1); NULL means every sequence holds n_kv.
  // n_kv stays the batch stride of K and V (the cache capacity).
  const int32_t* seq_len = nullptr;
  // K/V rows (kv.n_kv = n_kv for a contiguous cache, or a paged pool)
  KvRows kv;
};
int decode_n_split(int n_kv, int* keys_per_split);
hipError_t launch_attn_fwd_decode(const DecodePlan& p, hipStream_t st);
// bf16 / head_dim 128 split kernel (G <= 16); writes the partials and raw
// logits only, launch_attn_fwd_decode runs the combine
bool decode_uses_bf16_kernel(const Shape& s);
hipError_t launch_attn_decode_bf16(const DecodePlan& p, hipStream_t st);

// Decode score: S[b][j] = sum_h 2^(c * logit - m2) / l for candidate keys,
// from the raw logits (q.k) the decode pass stored.
struct DecodeScorePlan {
  int batch, h_q, h_kv, n_kv, n_cand;   // n_cand = candidates per row (p - window + 1)
  int window;
  float c;                        // softmax scale * log2(e)
  const float* logits; size_t logits_stride; const float* stats;
  float* scores; size_t score_stride;
  const int32_t* seq_len = nullptr;   // as in DecodePlan; n_cand then follows it
};
hipError_t launch_decode_score(const DecodeScorePlan& p, hipStream_t st);

// Pass 2 (prefill): head-summed probabilities for a chunk of queries of one
// sequence. Writes S[r][j] for r in [0, rows), j in [0, n_cand_max) where
// row r is query q0 + r; only j <= p - window are meaningful.
struct ScorePlan {
  Shape s;
  int b, q0, rows, window;
  const void* q; const void* k;
  const float* stats;
  float* scores; size_t score_stride;   // floats between rows
  // When nonzero, the row also holds, from float seg_off on, the maximum of
  // S over the candidate keys of each 64-key segment (segment s covers keys
  // [64 s, 64 s + 63]); written by the bf16 head-dim-128 kernel only.
  size_t seg_off = 0;
};
hipError_t launch_score_prefill(const ScorePlan& p, hipStream_t st);
// True when launch_score_prefill uses the bf16 head-dim-128 kernel (the one
// that writes segment maxima).
bool score_uses_bf16_kernel(const Shape& s);

// Selection for `rows` score rows: row r is flattened query flat0 + r
// (flattened query = b * n_q + i).
struct SelectPlan {
  int rows, flat0, n_q, n_kv;
  int top_k, window, width;
  bool block_mode; int block_size, top_blocks;
  const float* scores; size_t score_stride;
  size_t seg_off = 0;                 // segment maxima after each row (see ScorePlan), 0 = none
  int32_t* idx;                       // [batch, n_q, width]
  const int32_t* seq_len = nullptr;   // decode rows (n_q == 1): keys per sequence
};
hipError_t launch_select(const SelectPlan& p, hipStream_t st);

// Decode step over a growing cache: launch_set_lens writes `lens[i] + 1`
// (host values passed as kernel arguments) to seq_len[first + i];
// launch_kv_append then copies each sequence's new K and V row (row_bytes =
// h_kv * head_dim * element size, a multiple of 16) to position
// seq_len[b] - 1 of the caches [batch][cap][h_kv][head_dim].
hipError_t launch_set_lens(const int32_t* lens_host, int first, int count, int32_t* seq_len,
                           hipStream_t st);
hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* seq_len, int batch, const KvRows& kv, int row_bytes,
                            hipStream_t st);

// Chunked prefill over a paged pool. Sequence s of one launch (page-table
// row b[s]) visits positions r0[s] .. end[s] - 1 of its page list:
// positions at or past lens[s] are its new tokens (packed rows
// q0[s] + j - lens[s] of k_new / v_new), which land in the pool; when
// st0[s] >= 0 every visited row is also copied to row st0[s] + j of the
// contiguous staging buffers (new rows from k_new / v_new, older ones from
// the pool). Work-groups blk0[s] .. blk0[s+1] serve sequence s.
constexpr int STAGE_MAX_SEQS = 32;
constexpr int STAGE_ROWS = 8;               // positions per work-group
struct StageSeqs {
  int n = 0;
  int blk0[STAGE_MAX_SEQS + 1];
  int b[STAGE_MAX_SEQS], r0[STAGE_MAX_SEQS], end[STAGE_MAX_SEQS];
  int lens[STAGE_MAX_SEQS], q0[STAGE_MAX_SEQS];
  long long st0[STAGE_MAX_SEQS];
};
hipError_t launch_kv_stage(const StageSeqs& s, const void* k_new, const void* v_new, void* k_pool,
                           void* v_pool, void* k_stage, void* v_stage, const KvRows& kv,
                           int row_bytes, hipStream_t st);

// Copy one score row into a debug buffer: candidates keep S, others get -1.
hipError_t launch_export_scores(const float* src, int n_cand, int n_kv, float* dst,
                                hipStream_t st);

// Sparse layers over a given index set.
struct SparsePlan {
  const void* q; const void* k; const void* v;
  const int32_t* idx;
  void* o;
  int layers, batch, n_q, n_kv, h_q, h_kv, head_dim, width;
  float scale_log2;
  bool bf16;
  KvRows kv;                          // kv.n_kv = n_kv, or a paged pool
  size_t layer_stride = 0;            // elements between layers of q, o (0: batch*n_q*h_q*d)
};
hipError_t launch_sparse_attn(const SparsePlan& p, hipStream_t st);

// KV Bridging (bf16): k, v [tokens][features] = hidden [tokens][d_model] .
// w_kv[0 or 1]^T, w_kv [2 * features][d_model]; d_model a multiple of 64.
struct BridgePlan {
  const void* hidden; const void* w_kv;
  void* k; void* v;
  int tokens, features, d_model;
};
hipError_t launch_kv_bridge(const BridgePlan& p, hipStream_t st);

// Backward pass of the full layer: Delta = rowsum(dO * O) into `delta`
// ([batch][h_q][n_q] floats), then dK/dV and dQ, in that order on a stream. lse is the
// forward's natural-log LSE. acc_k / acc_v (nullable) hold the sparse
// layers' K/V gradient sums in the K/V layout, fp32, or with acc_fixed 64-bit
// fixed point to be multiplied by acc_scale[2] (K) and acc_scale[3] (V);
// they are added into dK, dV, so launch_sparse_bwd must run first on the
// same stream.
struct BwdPlan {
  Shape s;
  float scale;                         // softmax scale
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;
  float* delta;
  const void* acc_k; const void* acc_v;
  bool acc_fixed = false;
  const float* acc_scale = nullptr;
  void* dq; void* dk; void* dv;
  // bf16 / head_dim 128: K transposed to [batch][h_kv][tile][head_dim][64]
  // (as launch_v_transpose lays out V), read by the dQ kernel; NULL selects
  // the generic dQ kernel
  const void* kt = nullptr;
  // bf16 / head_dim 128: Q and dO transposed per (sequence, KV head, tile of
  // 64 rows) to [head_dim][64], and the tiles' rows' lse * log2(e) and Delta
  // ([tile][2][64]); written by launch_bwd_rows_layout, read by the dK/dV
  // kernel; NULL selects the generic dK/dV kernel
  void* qt = nullptr;
  void* dot = nullptr;
  float* rst = nullptr;
};
bool bwd_dq_uses_bf16_kernel(const Shape& s);
// tiles of the transposed row layout (each 64 x head_dim elements of qt and
// of dot, 128 floats of rst)
size_t bwd_rows_layout_tiles(const Shape& s);
hipError_t launch_bwd_rows_layout(const BwdPlan& p, hipStream_t st);   // after the delta
hipError_t launch_bwd_delta(const BwdPlan& p, hipStream_t st);
hipError_t launch_bwd_dkdv(const BwdPlan& p, hipStream_t st);   // after the delta
hipError_t launch_bwd_dq(const BwdPlan& p, hipStream_t st);     // after the delta

// Backward of `layers` sparse layers (layers * h_q / h_kv <= 64) over a
// fixed index set: writes dq and ADDS the K/V gradients into acc_k / acc_v
// ([batch][n_kv][h_kv][head_dim], zeroed by the caller) with atomics: fp32
// adds, or with `fixed` 64-bit integer adds of round(x * acc_scale[0]) (K)
// and round(x * acc_scale[1]) (V), whose sums do not depend on the order in
// which the adds land.
struct SparseBwdPlan {
  const void* q; const void* o; const void* dout;
  const void* k; const void* v;
  const int32_t* idx;
  void* dq;
  void* acc_k; void* acc_v;
  bool fixed = false;
  const float* acc_scale = nullptr;
  int layers, batch, n_q, n_kv, h_q, h_kv, head_dim, width;
  float scale, scale_log2;
  bool bf16;
};
hipError_t launch_sparse_bwd(const SparseBwdPlan& p, hipStream_t st);

// The fixed-point scales of the sparse layers' K/V sums, from bounds on what
// any sum can reach (every row's probabilities add up to one):
//   |dV| <= R max|dO|,   |dK| <= scale * 2 R max||dO|| max||V|| max|Q|,
// R = layers * n_q * h_q / h_kv rows per (sequence, KV head), norms over
// head-dim rows. Reads q / dout ([q_rows][head_dim], every sparse layer) and
// v ([v_rows][head_dim]) once; writes 4 maxima into `maxima` (zeroed by the
// caller) and scales[0..3] = 2^F_K, 2^F_V, 2^-F_K, 2^-F_V with the largest F
// that keeps every scaled sum below 2^61.
struct SparseBwdBoundPlan {
  const void* q; const void* dout; const void* v;
  size_t q_rows, v_rows;
  int head_dim;
  bool bf16;
  double rows;                         // R
  float scale;                         // softmax scale
  unsigned* maxima;
  float* scales;
};
hipError_t launch_sparse_bwd_bounds(const SparseBwdBoundPlan& p, hipStream_t st);

// p[0 .. n) = 0 (n a multiple of 4, p 16-byte aligned)
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st);

}  // namespace hs2
