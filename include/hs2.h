/*
 * hs2.h - C ABI of the HySparse2 Hybrid Block engine for AMD MI355X (gfx950).
 *
 * The Hybrid Block (HySparse2 pages: "Xiaomi Unveils HySparse2 for Faster
 * Long-Context AI", section "Two-Level KV Sharing"; openai-hub.net, section
 * "From Hybrid SWA to HySparse2") is one full-attention layer followed by
 * sparse-attention layers. The full layer produces the KV cache and decides
 * which tokens matter; the sparse layers reuse both (KV Reuse). Each sparse
 * layer attends, in one softmax, over the 128 most recent tokens plus 1024
 * tokens selected from outside that window (same page, section "Token-Level
 * Selection and Unified Local Access").
 *
 * Definitions used by every entry point (d = head_dim, G = h_q / h_kv):
 *   position of query i of sequence b:  p = n_kv - n_q + i
 *   KV head read by query head h:       g(h) = h / G  (integer division)
 *   logit:  s_h(p, j) = <Q[b,i,h,:], K[b,j,g(h),:]> * softmax_scale, j <= p
 *   full layer: causal softmax over j <= p; O = sum_j P_h(p, j) V[b,j,g(h),:]
 *   score:  S(p, j) = sum over all h_q heads of P_h(p, j)
 *   token selection: candidates j <= p - window; the min(top_k, #candidates)
 *       best by (-S, j) (ties go to the lower index), plus the window
 *       max(0, p - window + 1) .. p
 *   block selection (the previous generation's 64-token groups, bibibi.cc
 *       article, section "Article"): candidate blocks j / block_size scored by
 *       their max candidate score, best top_blocks by (-score, block), expanded
 *       to their candidate tokens, plus the window
 *   sparse layer l: softmax over the index set of query i, same K and V.
 *
 * Memory: every tensor pointer is a DEVICE pointer owned by the caller, in a
 * contiguous row-major layout, 16-byte aligned:
 *   Q, O           [batch, n_q, h_q, head_dim]        (dtype)
 *   K, V           [batch, n_kv, h_kv, head_dim]      (dtype), read only
 *   Q/O of layers  [n_layers, batch, n_q, h_q, head_dim]
 *   idx            [batch, n_q, hs2_index_width(p)]   int32; each row is the
 *                  strictly ascending index set followed by -1 padding
 *   lse            [batch, h_q, n_q] float, natural log (may be NULL)
 * The library allocates no device memory and keeps no state between calls.
 * Scratch space is the caller's workspace (size from hs2_workspace_size);
 * a smaller workspace only means more query chunks.
 *
 * Errors: arguments are checked on the host before anything is launched; a
 * non-OK status means nothing was written. HS2_ERR_DEVICE reports a HIP
 * launch failure; hs2_last_error() then holds the HIP error text (thread
 * local). No C++ exception crosses this interface. Non-finite inputs give
 * undefined results.
 *
 * Streams: every call is asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream); results are valid once the stream has synchronised. Calls
 * are reentrant when they use distinct workspaces.
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS2_ABI_VERSION 1

typedef enum {
  HS2_OK = 0,
  HS2_ERR_NULL = 1,         /* a required pointer is NULL                      */
  HS2_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes              */
  HS2_ERR_UNSUPPORTED = 3,  /* valid but not implemented (dtype, head_dim ...) */
  HS2_ERR_WORKSPACE = 4,    /* workspace smaller than the minimum              */
  HS2_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned                */
  HS2_ERR_DEVICE = 6        /* a HIP call failed                               */
} hs2_status;

typedef enum { HS2_FP32 = 0, HS2_BF16 = 1 } hs2_dtype;
typedef enum { HS2_SELECT_TOKEN = 0, HS2_SELECT_BLOCK = 1 } hs2_select;

/* One problem description shared by every call on the same block. */
typedef struct {
  int32_t abi_version;     /* must equal HS2_ABI_VERSION                       */
  int32_t dtype;           /* hs2_dtype of Q, K, V and every output tensor     */
  int32_t batch;           /* independent sequences, each with its own K/V     */
  int32_t n_q;             /* queries per sequence (1 = decode)                */
  int32_t n_kv;            /* keys per sequence; n_q <= n_kv                   */
  int32_t h_q, h_kv;       /* query heads and KV heads; h_q % h_kv == 0        */
  int32_t head_dim;        /* 64 or 128                                        */
  int32_t top_k;           /* selected tokens outside the window (1024)       */
  int32_t window;          /* always-kept recent tokens (128), >= 1            */
  int32_t select;          /* hs2_select                                       */
  int32_t block_size;      /* block mode only (64)                             */
  int32_t top_blocks;      /* block mode only (16)                             */
  float softmax_scale;     /* 1/sqrt(head_dim)                                 */
} hs2_problem;

/* Optional test hook: export the score rows of a few queries.
 * rows[r] is a flattened query (b * n_q + i); scores_out is a DEVICE buffer
 * [n_rows, n_kv] float that receives S(p, j) for the candidate keys
 * j <= p - window and -1 everywhere else. */
typedef struct {
  const int32_t* rows;     /* HOST array of n_rows flattened query indices     */
  int32_t n_rows;
  float* scores_out;       /* DEVICE [n_rows, n_kv]                            */
} hs2_debug;

/* ABI version compiled into the library. */
int32_t hs2_abi_version(void);

/* Width of one idx row: top_k + window (token mode) or
 * top_blocks * block_size + window (block mode); -1 if `p` is invalid. */
int32_t hs2_index_width(const hs2_problem* p);

/* Workspace needed by hs2_full_attn_select / hs2_block_forward.
 * *min_bytes lets the call run (one query row per chunk); *preferred_bytes
 * is what the library would use for the fastest schedule. Host only. */
hs2_status hs2_workspace_size(const hs2_problem* p, size_t* min_bytes,
                              size_t* preferred_bytes);

/* The full layer of the block: causal GQA attention (o), the per-head
 * log-sum-exp (lse, may be NULL), the head-summed scores and the selection
 * (idx). `dbg` may be NULL. */
hs2_status hs2_full_attn_select(const hs2_problem* p, const void* q,
                                const void* k, const void* v, void* o,
                                int32_t* idx, float* lse, const hs2_debug* dbg,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* n_layers sparse layers over a given index set (KV Reuse): layer l reads
 * q_layers[l] and writes o_layers[l]; every layer reads the same K, V and
 * idx. idx rows must be ascending, -1 padded, entries <= p. A row with no
 * entries (all -1) gives zero outputs. */
hs2_status hs2_sparse_attn(const hs2_problem* p, int32_t n_layers,
                           const void* q_layers, const void* k, const void* v,
                           const int32_t* idx, void* o_layers, void* stream);

/* The whole Hybrid Block: hs2_full_attn_select followed by n_sparse_layers
 * sparse layers that reuse its K/V and idx. */
hs2_status hs2_block_forward(const hs2_problem* p, int32_t n_sparse_layers,
                             const void* q_full, const void* q_sparse,
                             const void* k, const void* v, void* o_full,
                             void* o_sparse, int32_t* idx, float* lse,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * hs2_block_forward with its workspace taken from a buffer the library
 * holds in device memory, HS2_STATIC_WORKSPACE_BYTES on each GPU it runs
 * on, reserved when the library's device code is loaded onto that GPU and
 * held until the process ends. The call allocates nothing.
 *   Arguments, layouts and results are those of hs2_block_forward, without
 *   the workspace; the device is the calling thread's current HIP device.
 *   A problem whose minimum workspace (hs2_workspace_size) exceeds
 *   HS2_STATIC_WORKSPACE_BYTES returns HS2_ERR_WORKSPACE, like every other
 *   argument error, before any device call.
 *   Every call on one GPU uses that GPU's one buffer, which keeps what the
 *   last call left in it: calls on one GPU that overlap in time (on
 *   different streams, or from threads without ordering) race and give
 *   undefined results; calls ordered on one stream are safe. No part of the
 *   buffer has to start at zero (each pass writes what the next one reads),
 *   so nothing is cleared between calls. */
#define HS2_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
hs2_status hs2_block_forward_static(const hs2_problem* p, int32_t n_sparse_layers,
                                    const void* q_full, const void* q_sparse,
                                    const void* k, const void* v, void* o_full,
                                    void* o_sparse, int32_t* idx, float* lse,
                                    void* stream);

/* One decode step of the whole block over a growing KV cache, for a batch
 * of sequences of different lengths (the block's deployment shape: decode
 * is where the Cross-Decoder's hybrid blocks run, bound by memory bandwidth;
 * blog.lynxflow.co, section "Token-Level Sparse Selection and Deployment
 * Optimization"; the sparse layers reuse the one cache, hitechexpert.top,
 * section "Two-Level KV Sharing").
 *   p->n_q must be 1; p->n_kv is the cache capacity.
 *   k_cache, v_cache  DEVICE [batch, n_kv, h_kv, head_dim]: lens[b] valid rows
 *   k_new, v_new      DEVICE [batch, 1, h_kv, head_dim]: the new token's rows
 *   q_full            DEVICE [batch, 1, h_q, head_dim]
 *   q_sparse          DEVICE [n_sparse_layers, batch, 1, h_q, head_dim]
 *   lens              HOST [batch] lengths before the step, read during the
 *                     call only; 0 <= lens[b] < n_kv, else HS2_ERR_SHAPE
 *                     before any launch. The caller advances it.
 * The call writes k_new, v_new at row lens[b] of the caches, then runs the
 * block for the query at position lens[b] over keys 0..lens[b] (its own row
 * included): outputs as hs2_block_forward, idx entries are cache rows.
 * Workspace as hs2_workspace_size for the same problem. */
hs2_status hs2_decode_step(const hs2_problem* p, int32_t n_sparse_layers,
                           const void* q_full, const void* q_sparse,
                           const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* lens,
                           void* o_full, void* o_sparse, int32_t* idx,
                           float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* A paged KV pool: the K and V buffers are pools of n_pages pages of
 * page_size rows ([n_pages * page_size, h_kv, head_dim] each), and row j of
 * sequence b lives in page page_table[b * max_pages + j / page_size] at row
 * j % page_size. page_size is a power of two >= 32; the problem's n_kv must
 * equal max_pages * page_size (the longest a sequence may grow). Page ids
 * are read on the device and clamped to [0, n_pages): a bad id reads or
 * writes a wrong page of the pool, never memory outside it. */
typedef struct {
  const int32_t* page_table;   /* DEVICE [batch, max_pages]                  */
  int32_t page_size;
  int32_t max_pages;
  int32_t n_pages;
} hs2_kv_pages;

/* hs2_decode_step over a paged KV pool (serving layout for batched turns of
 * different lengths): k_pool, v_pool are the pools described by `pages`;
 * everything else as hs2_decode_step. idx entries are sequence positions
 * (not pool rows). HS2_ERR_SHAPE on a bad page geometry. */
hs2_status hs2_decode_step_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                 int32_t n_sparse_layers, const void* q_full,
                                 const void* q_sparse, const void* k_new,
                                 const void* v_new, void* k_pool, void* v_pool,
                                 const int32_t* lens, void* o_full, void* o_sparse,
                                 int32_t* idx, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* KV Bridging: the K and V a Cross-Decoder full layer reads are projections
 * of the hidden states of its Self-Decoder full layer (blog.lynxflow.co,
 * section "Architectural Innovation: Two-Level KV Sharing"; hitechexpert.top,
 * section "Two-Level KV Sharing"). Writes, for every token m of the batch,
 *   k[m, :] = hidden[m, :] . W_k^T,   v[m, :] = hidden[m, :] . W_v^T
 * straight into the [batch, n_kv, h_kv, head_dim] buffers every call above
 * reads. hidden DEVICE [batch, n_kv, d_model]; w_kv DEVICE
 * [2, h_kv * head_dim, d_model] (W_k then W_v, one row per output feature).
 * bf16 only (HS2_ERR_UNSUPPORTED otherwise), fp32 accumulation, results
 * rounded to bf16; d_model a positive multiple of 64. Uses only p's dtype,
 * batch, n_kv, h_kv and head_dim. */
hs2_status hs2_kv_bridge(const hs2_problem* p, int32_t d_model, const void* hidden,
                         const void* w_kv, void* k, void* v, void* stream);

/* Variable-length batches (batched agent turns: every sequence appends its
 * own number of new tokens to a context of its own length; hitechexpert.top,
 * section "Two-Level KV Sharing": the one shared cache serves all of a
 * sequence's layers). The batch is packed token-major:
 *   cu_q, cu_kv   HOST [batch + 1] int32 offsets, starting at 0 and not
 *                 decreasing; sequence b owns queries cu_q[b] .. cu_q[b+1]
 *                 and keys cu_kv[b] .. cu_kv[b+1], with
 *                 n_q(b) = cu_q[b+1] - cu_q[b] <= n_kv(b) = cu_kv[b+1] - cu_kv[b]
 *                 (query i of sequence b sits at position n_kv(b) - n_q(b) + i);
 *                 sequences with no query are skipped
 *   q_full, o_full  DEVICE [total_q, h_q, head_dim]
 *   q_sparse, o_sparse DEVICE [n_sparse_layers, total_q, h_q, head_dim]
 *   k, v            DEVICE [total_kv, h_kv, head_dim]
 *   idx             DEVICE [total_q, hs2_index_width(p)], key positions
 *                   within the sequence
 *   lse (nullable)  DEVICE float, sequence b's [h_q][n_q(b)] block at offset
 *                   h_q * cu_q[b]
 * p->batch is the number of sequences; p->n_q and p->n_kv are not used. Each
 * sequence is computed as hs2_block_forward with batch 1 and its own
 * lengths (one query: the decode path), one after another on `stream`,
 * sharing the workspace (hs2_workspace_size_varlen: the largest any
 * sequence needs). Every sequence's shape is checked before any launch. */
hs2_status hs2_workspace_size_varlen(const hs2_problem* p, const int32_t* cu_q,
                                     const int32_t* cu_kv, size_t* min_bytes,
                                     size_t* preferred_bytes);
hs2_status hs2_block_forward_varlen(const hs2_problem* p, int32_t n_sparse_layers,
                                    const int32_t* cu_q, const int32_t* cu_kv,
                                    const void* q_full, const void* q_sparse,
                                    const void* k, const void* v, void* o_full,
                                    void* o_sparse, int32_t* idx, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Chunked prefill over a paged KV pool (batched agent turns: each sequence
 * appends a chunk of new tokens, a user message or a tool result, after its
 * own cached context, and every layer of the block reads the one cache;
 * hitechexpert.top, section "Two-Level KV Sharing"). Pool and page table as
 * hs2_kv_pages; p->n_kv = pages->max_pages * pages->page_size is the
 * capacity of one sequence, p->batch the number of sequences, p->n_q unused.
 *   cu_q          HOST [batch + 1] int32 offsets from 0, not decreasing:
 *                 sequence b's n_q(b) new tokens are packed rows
 *                 cu_q[b] .. cu_q[b+1]
 *   lens          HOST [batch]: tokens sequence b holds before the call;
 *                 lens[b] + n_q(b) <= p->n_kv, else HS2_ERR_SHAPE before
 *                 any launch. The caller advances it.
 *   k_new, v_new  DEVICE [total_q, h_kv, head_dim]: the new tokens' rows
 *   q_full, o_full DEVICE [total_q, h_q, head_dim]
 *   q_sparse, o_sparse DEVICE [n_sparse_layers, total_q, h_q, head_dim]
 *   k_pool, v_pool DEVICE pools (written: the new rows land at positions
 *                 lens[b] .. lens[b] + n_q(b) - 1 of sequence b's pages)
 *   idx           DEVICE [total_q, hs2_index_width(p)]: positions within
 *                 the sequence
 *   lse (nullable) DEVICE float, as hs2_block_forward_varlen
 * The results are those of hs2_block_forward_varlen over the sequences'
 * logical K/V (n_kv(b) = lens[b] + n_q(b), query i at lens[b] + i). A
 * sequence with two or more new tokens is first copied, K and V rows 0 ..
 * n_kv(b) - 1, to contiguous staging buffers at the front of the workspace,
 * which its full layer, score pass and sparse layers then read: prefill is
 * bound by matrix math, and the copy is small beside it. A one-token
 * sequence reads the pool in place (the decode path); a batch of decode
 * steps alone is better served by hs2_decode_step_paged, one launch per pass
 * for all of them. Pages that a sequence's new tokens are written to must not
 * be read by another sequence of the same call (shared prefix pages may be).
 * Workspace: hs2_workspace_size_paged (16-byte aligned). */
hs2_status hs2_workspace_size_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                   const int32_t* cu_q, const int32_t* lens,
                                   size_t* min_bytes, size_t* preferred_bytes);
hs2_status hs2_block_forward_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                   int32_t n_sparse_layers, const int32_t* cu_q,
                                   const int32_t* lens, const void* q_full,
                                   const void* q_sparse, const void* k_new,
                                   const void* v_new, void* k_pool, void* v_pool,
                                   void* o_full, void* o_sparse, int32_t* idx,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Backward pass of the block, for fine-tuning (hitechexpert.top, section
 * "Performance Gains: Cost, Speed, and Long-Context Capabilities": the
 * compared models are fine-tuned alike). The index sets are held fixed (a
 * discrete selection passes no gradient back, so the score and selection
 * steps have none); the full layer and every sparse layer are
 * differentiated as softmax attention, and since they all read the one K/V
 * buffer (KV Reuse, section "Two-Level KV Sharing") their K/V gradients add:
 *   dK = dK_full + sum over layers dK_l,   dV likewise.
 * Inputs (DEVICE): everything hs2_block_forward read (q_full, q_sparse, k,
 * v) and wrote (o_full, o_sparse, idx, lse: the natural-log LSE, required),
 * plus the output gradients do_full [batch, n_q, h_q, head_dim] and do_sparse
 * [n_sparse_layers, batch, n_q, h_q, head_dim]. idx rows must be ascending,
 * -1 padded, entries <= p (as hs2_block_forward writes them).
 * Outputs (DEVICE, dtype, overwritten): dq_full, dq_sparse (shapes of
 * q_full, q_sparse), dk, dv (shape of k). Gradients are accumulated in fp32
 * and rounded once. The sparse layers' K/V sums use fp32 atomic adds, so
 * their last bits may differ from run to run (hs2_block_backward_deterministic
 * below avoids that); everything else is deterministic. With
 * n_sparse_layers = 0, q_sparse, o_sparse, idx, do_sparse and dq_sparse may
 * be NULL.
 * Workspace: hs2_backward_workspace_size bytes (Delta = rowsum(dO * O) per
 * row; for bf16 at head dim 128 a tiled K^T copy that the dQ kernel reads,
 * and Q and dO in transposed 64-row tiles with their rows' lse and Delta,
 * which the dK/dV kernel reads; the sparse layers' K/V accumulators, sized
 * for either entry point), 16-byte aligned. */
hs2_status hs2_backward_workspace_size(const hs2_problem* p, int32_t n_sparse_layers,
                                       size_t* bytes);
hs2_status hs2_block_backward(const hs2_problem* p, int32_t n_sparse_layers,
                              const void* q_full, const void* q_sparse,
                              const void* k, const void* v,
                              const void* o_full, const void* o_sparse,
                              const float* lse, const int32_t* idx,
                              const void* do_full, const void* do_sparse,
                              void* dq_full, void* dq_sparse, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream);

/* hs2_block_backward with bit-reproducible results: same arguments, same
 * workspace. The sparse layers' K/V sums are kept as 64-bit fixed point
 * (integer atomic adds, whose result does not depend on the order in which
 * they land) with a scale derived on the device from the inputs: a key's
 * sums over all rows of its KV head are bounded by R max|dO| (dV) and
 * softmax_scale * 2 R max||dO|| max||V|| max|Q| (dK), R the rows per
 * (sequence, KV head) over all sparse layers, and the scale is the largest
 * power of two that keeps those bounds below 2^61. The resolution is far
 * finer than fp32 sums keep (2^-39 for dV, 2^-34 for dK on a 32K-token
 * prefill with unit-variance inputs). Costs one extra read of q_sparse,
 * do_sparse and v, and 64-bit instead of 32-bit atomics. */
hs2_status hs2_block_backward_deterministic(const hs2_problem* p, int32_t n_sparse_layers,
                                            const void* q_full, const void* q_sparse,
                                            const void* k, const void* v,
                                            const void* o_full, const void* o_sparse,
                                            const float* lse, const int32_t* idx,
                                            const void* do_full, const void* do_sparse,
                                            void* dq_full, void* dq_sparse, void* dk, void* dv,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* Optional pass timing, a profiling aid. While enabled, every call records
 * HIP events on its stream around each pass: HS2_PASS_FULL (full attention,
 * pass 1), HS2_PASS_SCORE (head-summed scores, pass 2), HS2_PASS_SELECT
 * (selection), HS2_PASS_SPARSE (sparse layers), HS2_PASS_LAYOUT (the
 * copy of V into the workspace in key-tile-major transposed order that the
 * bf16 / head_dim 128 prefill kernel reads; absent on every other path),
 * the four HS2_PASS_BWD_* steps of hs2_block_backward, and HS2_PASS_KV_STAGE
 * (hs2_block_forward_paged's append and staging copy).
 * hs2_profile_enable(1)
 * starts a fresh record and (0) stops recording. hs2_profile_read waits for
 * the recorded events, then writes the summed milliseconds and the number of
 * timed launches of each pass (arrays of HS2_N_PASSES) and clears the record.
 * Process-wide state; not meant for concurrent profiled calls. */
typedef enum {
  HS2_PASS_FULL = 0,
  HS2_PASS_SCORE = 1,
  HS2_PASS_SELECT = 2,
  HS2_PASS_SPARSE = 3,
  HS2_PASS_LAYOUT = 4,
  HS2_PASS_BWD_PREP = 5,    /* backward: Delta, K^T and Q/dO tile copies,
                               accumulators cleared                        */
  HS2_PASS_BWD_SPARSE = 6,  /* backward: the sparse layers                   */
  HS2_PASS_BWD_DKDV = 7,    /* backward: the full layer's dK, dV             */
  HS2_PASS_BWD_DQ = 8,      /* backward: the full layer's dQ                 */
  HS2_PASS_KV_STAGE = 9,    /* paged prefill: new rows in, staging copies    */
  HS2_N_PASSES = 10
} hs2_pass;
hs2_status hs2_profile_enable(int32_t on);
hs2_status hs2_profile_read(double* ms, int64_t* launches);

/* Static text for a status code. */
const char* hs2_status_string(hs2_status s);

/* Detail for the last non-OK status returned on this thread ("" if none). */
const char* hs2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H */
