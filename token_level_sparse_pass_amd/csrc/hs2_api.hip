// C ABI of the Hybrid Block engine (declared in include/hs2.h): argument
// checks, workspace planning, query chunking and kernel launches. The block
// is one full-attention layer whose KV cache and token selection are reused
// by the sparse layers that follow (HySparse2 pages: "Xiaomi Unveils
// HySparse2 for Faster Long-Context AI", section "Two-Level KV Sharing").
//
// Every check runs on the host before the first launch; nothing is written
// when a call returns an error. No C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <cstring>
#include <string>
#include <mutex>
#include <vector>

#include "hs2.h"
#include "hs2_launch.h"

namespace {

thread_local std::string g_err;

hs2_status fail(hs2_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hs2_status fail(hs2_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

hs2_status device_fail(hipError_t e, const char* what) {
  return fail(HS2_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
constexpr int TOPK_MAX = 4096;            // radix select list capacity
constexpr int MAX_BLOCKS = 16384;         // block mode: blocks per score row
constexpr int MAX_TOP_BLOCKS = 256;
constexpr size_t CHUNK_TARGET = (size_t)4 << 30;   // preferred score chunk, bytes

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool is_decode(const hs2_problem& p) { return p.n_q == 1; }

int index_width(const hs2_problem& p) {
  return p.select == HS2_SELECT_TOKEN ? p.top_k + p.window : p.top_blocks * p.block_size + p.window;
}

// longest score row (candidates of the last query), padded to 256 floats
size_t score_stride(const hs2_problem& p) {
  const long long n = (long long)p.n_kv - p.window;
  return n > 0 ? (size_t)((n + 255) / 256 * 256) : 0;
}

hs2_status check_problem(const hs2_problem* p) {
  if (!p) return fail(HS2_ERR_NULL, "problem is NULL");
  if (p->abi_version != HS2_ABI_VERSION)
    return fail(HS2_ERR_UNSUPPORTED, "abi_version %d, library has %d", p->abi_version,
                HS2_ABI_VERSION);
  if (p->dtype != HS2_FP32 && p->dtype != HS2_BF16)
    return fail(HS2_ERR_UNSUPPORTED, "dtype %d", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HS2_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", p->head_dim);
  if (p->batch < 1 || p->n_q < 1 || p->n_kv < 1)
    return fail(HS2_ERR_SHAPE, "batch %d, n_q %d, n_kv %d must be >= 1", p->batch, p->n_q, p->n_kv);
  if (p->n_q > p->n_kv) return fail(HS2_ERR_SHAPE, "n_q %d > n_kv %d", p->n_q, p->n_kv);
  if (p->h_q < 1 || p->h_kv < 1 || p->h_q % p->h_kv != 0)
    return fail(HS2_ERR_SHAPE, "h_q %d must be a positive multiple of h_kv %d", p->h_q, p->h_kv);
  const int G = p->h_q / p->h_kv;
  if (G > 64) return fail(HS2_ERR_UNSUPPORTED, "h_q / h_kv = %d > 64", G);
  if (p->n_q == 1 && G > 32)
    return fail(HS2_ERR_UNSUPPORTED, "decode with h_q / h_kv = %d > 32", G);
  if (p->window < 1) return fail(HS2_ERR_SHAPE, "window %d must be >= 1", p->window);
  if (p->select != HS2_SELECT_TOKEN && p->select != HS2_SELECT_BLOCK)
    return fail(HS2_ERR_UNSUPPORTED, "select %d", p->select);
  if (p->select == HS2_SELECT_TOKEN) {
    if (p->top_k < 0 || p->top_k > TOPK_MAX)
      return fail(HS2_ERR_UNSUPPORTED, "top_k %d (0..%d)", p->top_k, TOPK_MAX);
  } else {
    if (p->block_size < 1) return fail(HS2_ERR_SHAPE, "block_size %d", p->block_size);
    if (p->top_blocks < 1 || p->top_blocks > MAX_TOP_BLOCKS)
      return fail(HS2_ERR_UNSUPPORTED, "top_blocks %d (1..%d)", p->top_blocks, MAX_TOP_BLOCKS);
    const long long nb = ((long long)p->n_kv - p->window + p->block_size - 1) / p->block_size;
    if (nb > MAX_BLOCKS)
      return fail(HS2_ERR_UNSUPPORTED, "%lld candidate blocks per row > %d", nb, MAX_BLOCKS);
  }
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale))
    return fail(HS2_ERR_SHAPE, "softmax_scale must be positive and finite");
  // element offsets of every tensor must fit the kernels' 64-bit math, and
  // per-sequence key/row counts their 32-bit math
  const long long w = index_width(*p);
  if (w < 1 || w > (1 << 20)) return fail(HS2_ERR_SHAPE, "index width %lld", w);
  if ((long long)p->n_q * G * 2 > (1LL << 31) || (long long)p->batch * p->n_q > (1LL << 31) / w)
    return fail(HS2_ERR_SHAPE, "too many query rows");
  return HS2_OK;
}

hs2::Shape shape_of(const hs2_problem& p) {
  hs2::Shape s;
  s.batch = p.batch; s.n_q = p.n_q; s.n_kv = p.n_kv; s.h_q = p.h_q; s.h_kv = p.h_kv;
  s.head_dim = p.head_dim; s.bf16 = p.dtype == HS2_BF16;
  s.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  return s;
}

struct Layout {
  size_t stats = 0;          // [3][B][h_q][n_q] floats: m2, l, 1/l
  size_t vt = 0;             // transposed V (bf16, head_dim 128 prefill), 0 = none
  int vt_keys = 0;
  size_t part = 0, logits = 0, scores = 0;   // byte offsets
  size_t n_part = 0, n_logits = 0;
  size_t logits_stride = 0;  // floats per logits row (decode)
  size_t lens = 0;           // [B] int32 keys per sequence (decode step)
  size_t stride = 0;         // floats per score row
  size_t seg_off = 0;        // prefill: float offset of the segment maxima in a row, 0 = none
  int chunk_rows = 0;        // prefill query rows per chunk
  int n_split = 0, kps = 0;  // decode split
  size_t total = 0;
};

// Workspace layout for `ws_bytes` available (SIZE_MAX = plan the preferred).
hs2_status plan(const hs2_problem& p, size_t ws_bytes, Layout* L, size_t* min_bytes,
                size_t* pref_bytes) {
  Layout l;
  l.stride = score_stride(p);
  const size_t stats_b = align_up((size_t)3 * p.batch * p.h_q * p.n_q * sizeof(float));
  l.stats = 0;
  size_t off = stats_b;
  if (is_decode(p)) {
    l.n_split = hs2::decode_n_split(p.n_kv, &l.kps);
    l.part = off;
    l.n_part = (size_t)p.batch * p.h_q * l.n_split * (p.head_dim + 2);
    off += align_up(l.n_part * sizeof(float));
    l.logits = off;
    l.logits_stride = ((size_t)p.n_kv + 63) / 64 * 64;
    l.n_logits = (size_t)p.batch * p.h_q * l.logits_stride;
    off += align_up(l.n_logits * sizeof(float));
    l.scores = off;
    off += align_up((size_t)p.batch * std::max<size_t>(l.stride, 1) * sizeof(float));
    l.lens = off;
    off += align_up((size_t)p.batch * sizeof(int32_t));
    l.chunk_rows = p.batch;
    l.total = off;
    if (min_bytes) *min_bytes = off;
    if (pref_bytes) *pref_bytes = off;
  } else {
    if (hs2::prefill_uses_vt(shape_of(p))) {
      l.vt_keys = hs2::vt_keys_for(p.n_kv);
      l.vt = off;
      off += align_up((size_t)p.batch * p.h_kv * p.head_dim * l.vt_keys * 2);
    }
    l.scores = off;
    if (hs2::score_uses_bf16_kernel(shape_of(p)) && l.stride >= 256) {
      // each row carries the maxima of its 64-key segments after the scores
      l.seg_off = l.stride;
      l.stride += l.stride / 64;
    }
    const size_t row_b = std::max<size_t>(l.stride, 1) * sizeof(float);
    const size_t mn = off + align_up(row_b);
    // the preferred chunk holds CHUNK_TARGET bytes of scores (the segment
    // maxima come on top of it)
    const size_t score_b = std::max<size_t>(l.seg_off ? l.seg_off : l.stride, 1) * sizeof(float);
    size_t pref_rows = std::max<size_t>(128, CHUNK_TARGET / score_b / 128 * 128);
    pref_rows = std::min<size_t>(pref_rows, ((size_t)p.n_q + 127) / 128 * 128);
    const size_t pref = off + align_up(pref_rows * row_b);
    if (min_bytes) *min_bytes = mn;
    if (pref_bytes) *pref_bytes = pref;
    if (ws_bytes != SIZE_MAX) {
      if (ws_bytes < mn) return HS2_ERR_WORKSPACE;
      size_t rows = (ws_bytes - off) / row_b;
      if (rows >= 128) rows = rows / 128 * 128;
      rows = std::min<size_t>(rows, (size_t)p.n_q);
      l.chunk_rows = (int)std::max<size_t>(rows, 1);
      l.total = off + align_up((size_t)l.chunk_rows * row_b);
    }
  }
  if (L) *L = l;
  return HS2_OK;
}

// ---- optional pass timing --------------------------------------------------
struct TimedPass {
  int pass;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedPass> g_prof;

// Records an event pair around one pass when profiling is on.
struct PassTimer {
  hipStream_t st;
  int pass;
  hipEvent_t start = nullptr, stop = nullptr;
  PassTimer(hipStream_t s, int p) : st(s), pass(p) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    if (hipEventCreate(&start) != hipSuccess || hipEventCreate(&stop) != hipSuccess) {
      start = stop = nullptr;
      return;
    }
    (void)hipEventRecord(start, st);
  }
  ~PassTimer() {
    if (!start) return;
    (void)hipEventRecord(stop, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({pass, start, stop});
  }
};

float* fptr(void* ws, size_t off) { return reinterpret_cast<float*>((char*)ws + off); }


hs2_status check_ptr(const void* ptr, const char* name, bool required = true) {
  if (!ptr) return required ? fail(HS2_ERR_NULL, "%s is NULL", name) : HS2_OK;
  if (!aligned16(ptr)) return fail(HS2_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return HS2_OK;
}

#define HS2_TRY(expr)                  \
  do {                                 \
    const hs2_status s_ = (expr);      \
    if (s_ != HS2_OK) return s_;       \
  } while (0)

#define HIP_TRY(expr, what)                        \
  do {                                             \
    const hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return device_fail(e_, what); \
  } while (0)

hs2_status check_full_args(const hs2_problem* p, const void* q, const void* k, const void* v,
                           const void* o, const int32_t* idx, const float* lse,
                           const hs2_debug* dbg, const void* ws, size_t ws_bytes,
                           Layout* layout) {
  HS2_TRY(check_problem(p));
  HS2_TRY(check_ptr(q, "q"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  HS2_TRY(check_ptr(o, "o"));
  HS2_TRY(check_ptr(idx, "idx"));
  HS2_TRY(check_ptr(lse, "lse", false));
  size_t mn = 0;
  if (plan(*p, SIZE_MAX, nullptr, &mn, nullptr) != HS2_OK) return fail(HS2_ERR_SHAPE, "plan");
  if (!ws) return fail(HS2_ERR_NULL, "workspace is NULL (needs %zu bytes)", mn);
  if (!aligned16(ws)) return fail(HS2_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < mn) return fail(HS2_ERR_WORKSPACE, "workspace %zu bytes < minimum %zu", ws_bytes, mn);
  if (plan(*p, ws_bytes, layout, nullptr, nullptr) != HS2_OK)
    return fail(HS2_ERR_WORKSPACE, "workspace too small");
  if (dbg) {
    if (dbg->n_rows < 0) return fail(HS2_ERR_SHAPE, "debug n_rows %d", dbg->n_rows);
    if (dbg->n_rows > 0) {
      if (!dbg->rows) return fail(HS2_ERR_NULL, "debug rows is NULL");
      if (!dbg->scores_out) return fail(HS2_ERR_NULL, "debug scores_out is NULL");
      for (int r = 0; r < dbg->n_rows; ++r)
        if (dbg->rows[r] < 0 || (long long)dbg->rows[r] >= (long long)p->batch * p->n_q)
          return fail(HS2_ERR_SHAPE, "debug row %d out of range", dbg->rows[r]);
    }
  }
  return HS2_OK;
}

hs2::KvRows contiguous_rows(const hs2_problem& p) {
  hs2::KvRows kv;
  kv.n_kv = p.n_kv;
  return kv;
}

// seq_len (decode only, device, may be NULL): keys held by each sequence,
// whose query then sits at seq_len[b] - 1; NULL means n_kv for all.
// kv (decode only, may be NULL): where K/V rows live; NULL = contiguous.
hs2_status run_full(const hs2_problem& p, const void* q, const void* k, const void* v, void* o,
                    int32_t* idx, float* lse, const hs2_debug* dbg, void* ws,
                    const Layout& L, hipStream_t st, const int32_t* seq_len = nullptr,
                    const hs2::KvRows* kv = nullptr) {
  const hs2::Shape s = shape_of(p);
  float* stats = fptr(ws, L.stats);
  float* scores = fptr(ws, L.scores);
  const int width = index_width(p);
  const bool block_mode = p.select == HS2_SELECT_BLOCK;

  auto export_rows = [&](int flat_lo, int flat_hi) -> hs2_status {
    if (!dbg) return HS2_OK;
    for (int r = 0; r < dbg->n_rows; ++r) {
      const int f = dbg->rows[r];
      if (f < flat_lo || f >= flat_hi) continue;
      const int i = f % p.n_q;
      const int n_c = std::max(0, p.n_kv - p.n_q + i - p.window + 1);
      HIP_TRY(hs2::launch_export_scores(scores + (size_t)(f - flat_lo) * L.stride, n_c, p.n_kv,
                                        dbg->scores_out + (size_t)r * p.n_kv, st),
              "export scores");
    }
    return HS2_OK;
  };

  if (is_decode(p)) {
    hs2::DecodePlan d;
    d.s = s; d.q = q; d.k = k; d.v = v; d.o = o; d.stats = stats; d.lse = lse;
    d.part = fptr(ws, L.part); d.logits = fptr(ws, L.logits); d.logits_stride = L.logits_stride;
    d.keys_per_split = L.kps; d.n_split = L.n_split; d.seq_len = seq_len;
    d.kv = kv ? *kv : contiguous_rows(p);
    {
      PassTimer t(st, HS2_PASS_FULL);
      HIP_TRY(hs2::launch_attn_fwd_decode(d, st), "decode attention");
    }
    hs2::DecodeScorePlan ds;
    ds.batch = p.batch; ds.h_q = p.h_q; ds.h_kv = p.h_kv; ds.n_kv = p.n_kv; ds.c = s.scale_log2;
    ds.n_cand = std::max(0, p.n_kv - p.window);
    ds.window = p.window; ds.seq_len = seq_len;
    ds.logits = d.logits; ds.logits_stride = L.logits_stride; ds.stats = stats; ds.scores = scores; ds.score_stride = L.stride;
    {
      PassTimer t(st, HS2_PASS_SCORE);
      HIP_TRY(hs2::launch_decode_score(ds, st), "decode score");
    }
    HS2_TRY(export_rows(0, p.batch));
    hs2::SelectPlan sp;
    sp.rows = p.batch; sp.flat0 = 0; sp.n_q = 1; sp.n_kv = p.n_kv; sp.seq_len = seq_len;
    sp.top_k = p.top_k; sp.window = p.window; sp.width = width;
    sp.block_mode = block_mode; sp.block_size = p.block_size; sp.top_blocks = p.top_blocks;
    sp.scores = scores; sp.score_stride = L.stride; sp.idx = idx;
    {
      PassTimer t(st, HS2_PASS_SELECT);
      HIP_TRY(hs2::launch_select(sp, st), "select");
    }
    return HS2_OK;
  }

  hs2::FwdPlan f;
  f.s = s; f.q = q; f.k = k; f.v = v; f.o = o; f.stats = stats; f.lse = lse;
  f.vt = L.vt ? (char*)ws + L.vt : nullptr;
  f.vt_keys = L.vt_keys;
  if (f.vt) {
    PassTimer t(st, HS2_PASS_LAYOUT);
    HIP_TRY(hs2::launch_v_transpose(f, st), "V transpose");
  }
  {
    PassTimer t(st, HS2_PASS_FULL);
    HIP_TRY(hs2::launch_attn_fwd_prefill(f, st), "full attention");
  }
  for (int b = 0; b < p.batch; ++b) {
    for (int q0 = 0; q0 < p.n_q; q0 += L.chunk_rows) {
      const int rows = std::min(L.chunk_rows, p.n_q - q0);
      hs2::ScorePlan sc;
      sc.s = s; sc.b = b; sc.q0 = q0; sc.rows = rows; sc.window = p.window;
      sc.q = q; sc.k = k; sc.stats = stats; sc.scores = scores; sc.score_stride = L.stride;
      sc.seg_off = L.seg_off;
      {
        PassTimer t(st, HS2_PASS_SCORE);
        HIP_TRY(hs2::launch_score_prefill(sc, st), "score");
      }
      const int flat0 = b * p.n_q + q0;
      HS2_TRY(export_rows(flat0, flat0 + rows));
      hs2::SelectPlan sp;
      sp.rows = rows; sp.flat0 = flat0; sp.n_q = p.n_q; sp.n_kv = p.n_kv;
      sp.top_k = p.top_k; sp.window = p.window; sp.width = width;
      sp.block_mode = block_mode; sp.block_size = p.block_size; sp.top_blocks = p.top_blocks;
      sp.scores = scores; sp.score_stride = L.stride; sp.seg_off = L.seg_off; sp.idx = idx;
      {
        PassTimer t(st, HS2_PASS_SELECT);
        HIP_TRY(hs2::launch_select(sp, st), "select");
      }
    }
  }
  return HS2_OK;
}

hs2_status check_sparse_args(const hs2_problem* p, int32_t n_layers, const void* q, const void* k,
                             const void* v, const int32_t* idx, const void* o) {
  HS2_TRY(check_problem(p));
  if (n_layers < 0) return fail(HS2_ERR_SHAPE, "n_layers %d", n_layers);
  if (n_layers == 0) return HS2_OK;
  HS2_TRY(check_ptr(q, "q_layers"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  HS2_TRY(check_ptr(idx, "idx"));
  HS2_TRY(check_ptr(o, "o_layers"));
  return HS2_OK;
}

// layer_elems: elements between layers of q and o (0: batch * n_q * h_q * d)
hs2_status run_sparse(const hs2_problem& p, int32_t n_layers, const void* q, const void* k,
                      const void* v, const int32_t* idx, void* o, hipStream_t st,
                      const hs2::KvRows* kv = nullptr, size_t layer_elems = 0) {
  const int G = p.h_q / p.h_kv;
  const int per = std::max(1, 64 / G);                       // layers per launch
  const size_t esz = p.dtype == HS2_BF16 ? 2 : 4;
  if (layer_elems == 0) layer_elems = (size_t)p.batch * p.n_q * p.h_q * p.head_dim;
  for (int l0 = 0; l0 < n_layers; l0 += per) {
    hs2::SparsePlan sp;
    sp.layers = std::min(per, n_layers - l0);
    sp.q = (const char*)q + l0 * layer_elems * esz;
    sp.o = (char*)o + l0 * layer_elems * esz;
    sp.k = k; sp.v = v; sp.idx = idx;
    sp.batch = p.batch; sp.n_q = p.n_q; sp.n_kv = p.n_kv; sp.h_q = p.h_q; sp.h_kv = p.h_kv;
    sp.head_dim = p.head_dim; sp.width = index_width(p);
    sp.scale_log2 = p.softmax_scale * 1.4426950408889634f;
    sp.bf16 = p.dtype == HS2_BF16;
    sp.kv = kv ? *kv : contiguous_rows(p);
    sp.layer_stride = layer_elems;
    PassTimer t(st, HS2_PASS_SPARSE);
    HIP_TRY(hs2::launch_sparse_attn(sp, st), "sparse attention");
  }
  return HS2_OK;
}

}  // namespace

extern "C" {

int32_t hs2_abi_version(void) { return HS2_ABI_VERSION; }

int32_t hs2_index_width(const hs2_problem* p) {
  if (check_problem(p) != HS2_OK) return -1;
  return index_width(*p);
}

hs2_status hs2_workspace_size(const hs2_problem* p, size_t* min_bytes, size_t* preferred_bytes) {
  g_err.clear();
  HS2_TRY(check_problem(p));
  if (!min_bytes && !preferred_bytes) return fail(HS2_ERR_NULL, "no output pointer");
  return plan(*p, SIZE_MAX, nullptr, min_bytes, preferred_bytes);
}

hs2_status hs2_full_attn_select(const hs2_problem* p, const void* q, const void* k, const void* v,
                                void* o, int32_t* idx, float* lse, const hs2_debug* dbg,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  Layout L;
  HS2_TRY(check_full_args(p, q, k, v, o, idx, lse, dbg, workspace, workspace_bytes, &L));
  return run_full(*p, q, k, v, o, idx, lse, dbg, workspace, L, (hipStream_t)stream);
}

hs2_status hs2_sparse_attn(const hs2_problem* p, int32_t n_layers, const void* q_layers,
                           const void* k, const void* v, const int32_t* idx, void* o_layers,
                           void* stream) {
  g_err.clear();
  HS2_TRY(check_sparse_args(p, n_layers, q_layers, k, v, idx, o_layers));
  if (n_layers == 0) return HS2_OK;
  return run_sparse(*p, n_layers, q_layers, k, v, idx, o_layers, (hipStream_t)stream);
}

hs2_status hs2_block_forward(const hs2_problem* p, int32_t n_sparse_layers, const void* q_full,
                             const void* q_sparse, const void* k, const void* v, void* o_full,
                             void* o_sparse, int32_t* idx, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err.clear();
  Layout L;
  HS2_TRY(check_full_args(p, q_full, k, v, o_full, idx, lse, nullptr, workspace, workspace_bytes,
                          &L));
  HS2_TRY(check_sparse_args(p, n_sparse_layers, q_sparse, k, v, idx, o_sparse));
  const hipStream_t st = (hipStream_t)stream;
  HS2_TRY(run_full(*p, q_full, k, v, o_full, idx, lse, nullptr, workspace, L, st));
  if (n_sparse_layers == 0) return HS2_OK;
  return run_sparse(*p, n_sparse_layers, q_sparse, k, v, idx, o_sparse, st);
}

}  // extern "C"

namespace {

// The workspace of hs2_block_forward_static: one copy of this array on each
// GPU the library runs on. In host code its name is only a stand-in, so the
// device address of each GPU's copy is looked up once, with that GPU
// current, and every launch receives that address.
static __device__ __align__(256) char scratch[HS2_STATIC_WORKSPACE_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

hs2_status scratch_of_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(HS2_ERR_DEVICE, "device %d: the static workspace serves devices 0..%d", dev,
                MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "static workspace address");
    if (!ptr) return fail(HS2_ERR_DEVICE, "static workspace has no device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HS2_OK;
}

}  // namespace

extern "C" {

hs2_status hs2_block_forward_static(const hs2_problem* p, int32_t n_sparse_layers,
                                    const void* q_full, const void* q_sparse, const void* k,
                                    const void* v, void* o_full, void* o_sparse, int32_t* idx,
                                    float* lse, void* stream) {
  g_err.clear();
  // every host check first: nothing touches a device before they pass
  HS2_TRY(check_problem(p));
  size_t mn = 0;
  if (plan(*p, SIZE_MAX, nullptr, &mn, nullptr) != HS2_OK) return fail(HS2_ERR_SHAPE, "plan");
  if (mn > HS2_STATIC_WORKSPACE_BYTES)
    return fail(HS2_ERR_WORKSPACE,
                "the problem needs a workspace of at least %zu bytes; the static one holds %zu",
                mn, (size_t)HS2_STATIC_WORKSPACE_BYTES);
  HS2_TRY(check_ptr(q_full, "q_full"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  HS2_TRY(check_ptr(o_full, "o_full"));
  HS2_TRY(check_ptr(idx, "idx"));
  HS2_TRY(check_ptr(lse, "lse", false));
  HS2_TRY(check_sparse_args(p, n_sparse_layers, q_sparse, k, v, idx, o_sparse));
  void* ws = nullptr;
  HS2_TRY(scratch_of_current_device(&ws));
  return hs2_block_forward(p, n_sparse_layers, q_full, q_sparse, k, v, o_full, o_sparse, idx, lse,
                           ws, HS2_STATIC_WORKSPACE_BYTES, stream);
}

namespace {

// A paged pool's geometry; p.n_kv must be its per-sequence capacity.
hs2_status check_pages(const hs2_problem& p, const hs2_kv_pages* pages, hs2::KvRows* kv) {
  if (!pages) return fail(HS2_ERR_NULL, "pages is NULL");
  if (!pages->page_table) return fail(HS2_ERR_NULL, "page_table is NULL");
  const int ps = pages->page_size;
  if (ps < 32 || (ps & (ps - 1)))
    return fail(HS2_ERR_SHAPE, "page_size %d: a power of two >= 32 is needed", ps);
  if (pages->max_pages < 1 || pages->n_pages < 1)
    return fail(HS2_ERR_SHAPE, "max_pages %d, n_pages %d", pages->max_pages, pages->n_pages);
  if ((long long)pages->max_pages * ps != p.n_kv)
    return fail(HS2_ERR_SHAPE, "n_kv %d must be max_pages * page_size = %lld", p.n_kv,
                (long long)pages->max_pages * ps);
  if ((long long)pages->n_pages * ps > INT32_MAX)
    return fail(HS2_ERR_UNSUPPORTED, "pool of %d pages of %d rows", pages->n_pages, ps);
  *kv = contiguous_rows(p);
  kv->table = pages->page_table;
  kv->page_shift = __builtin_ctz((unsigned)ps);
  kv->max_pages = pages->max_pages;
  kv->n_pages = pages->n_pages;
  return HS2_OK;
}

// Shared by the contiguous and paged decode steps: validate, set the
// per-sequence key counts, append the new rows, run the block.
hs2_status decode_step_impl(const hs2_problem* p, const hs2_kv_pages* pages,
                            int32_t n_sparse_layers, const void* q_full, const void* q_sparse,
                            const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* lens, void* o_full, void* o_sparse, int32_t* idx,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  HS2_TRY(check_problem(p));
  if (p->n_q != 1) return fail(HS2_ERR_SHAPE, "a decode step has one query per sequence (n_q %d)",
                               p->n_q);
  hs2::KvRows kv = contiguous_rows(*p);
  if (pages) HS2_TRY(check_pages(*p, pages, &kv));
  if (!lens) return fail(HS2_ERR_NULL, "lens is NULL");
  for (int b = 0; b < p->batch; ++b)
    if (lens[b] < 0 || lens[b] >= p->n_kv)
      return fail(HS2_ERR_SHAPE, "lens[%d] = %d: a cache of %d keys has no room for one more", b,
                  lens[b], p->n_kv);
  HS2_TRY(check_ptr(k_new, "k_new"));
  HS2_TRY(check_ptr(v_new, "v_new"));
  Layout L;
  HS2_TRY(check_full_args(p, q_full, k_cache, v_cache, o_full, idx, lse, nullptr, workspace,
                          workspace_bytes, &L));
  HS2_TRY(check_sparse_args(p, n_sparse_layers, q_sparse, k_cache, v_cache, idx, o_sparse));
  const hipStream_t st = (hipStream_t)stream;
  int32_t* seq_len = reinterpret_cast<int32_t*>((char*)workspace + L.lens);
  const int row_bytes = p->h_kv * p->head_dim * (p->dtype == HS2_BF16 ? 2 : 4);
  HIP_TRY(hs2::launch_set_lens(lens, 0, p->batch, seq_len, st), "sequence lengths");
  HIP_TRY(hs2::launch_kv_append(k_new, v_new, k_cache, v_cache, seq_len, p->batch, kv, row_bytes,
                                st),
          "KV append");
  HS2_TRY(run_full(*p, q_full, k_cache, v_cache, o_full, idx, lse, nullptr, workspace, L, st,
                   seq_len, &kv));
  if (n_sparse_layers == 0) return HS2_OK;
  return run_sparse(*p, n_sparse_layers, q_sparse, k_cache, v_cache, idx, o_sparse, st, &kv);
}

}  // namespace

hs2_status hs2_decode_step(const hs2_problem* p, int32_t n_sparse_layers, const void* q_full,
                           const void* q_sparse, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* lens, void* o_full,
                           void* o_sparse, int32_t* idx, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err.clear();
  return decode_step_impl(p, nullptr, n_sparse_layers, q_full, q_sparse, k_new, v_new, k_cache,
                          v_cache, lens, o_full, o_sparse, idx, lse, workspace, workspace_bytes,
                          stream);
}

hs2_status hs2_decode_step_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                 int32_t n_sparse_layers, const void* q_full,
                                 const void* q_sparse, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, const int32_t* lens, void* o_full,
                                 void* o_sparse, int32_t* idx, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!pages) return fail(HS2_ERR_NULL, "pages is NULL");
  return decode_step_impl(p, pages, n_sparse_layers, q_full, q_sparse, k_new, v_new, k_pool,
                          v_pool, lens, o_full, o_sparse, idx, lse, workspace, workspace_bytes,
                          stream);
}

hs2_status hs2_kv_bridge(const hs2_problem* p, int32_t d_model, const void* hidden,
                         const void* w_kv, void* k, void* v, void* stream) {
  g_err.clear();
  HS2_TRY(check_problem(p));
  if (p->dtype != HS2_BF16) return fail(HS2_ERR_UNSUPPORTED, "KV bridging is bf16 only");
  if (d_model <= 0 || d_model % 64)
    return fail(HS2_ERR_SHAPE, "d_model %d: a positive multiple of 64 is needed", d_model);
  const long long tokens = (long long)p->batch * p->n_kv;
  if (tokens > INT32_MAX) return fail(HS2_ERR_UNSUPPORTED, "%lld tokens", tokens);
  HS2_TRY(check_ptr(hidden, "hidden"));
  HS2_TRY(check_ptr(w_kv, "w_kv"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  hs2::BridgePlan b;
  b.hidden = hidden; b.w_kv = w_kv; b.k = k; b.v = v;
  b.tokens = (int)tokens; b.features = p->h_kv * p->head_dim; b.d_model = d_model;
  HIP_TRY(hs2::launch_kv_bridge(b, (hipStream_t)stream), "KV bridge");
  return HS2_OK;
}

}  // extern "C"

namespace {

// Backward workspace: Delta [B][h_q][n_q] floats; for bf16 / head_dim 128
// the transposed K copy the dQ kernel reads ([B][h_kv][tile][d][64 keys]);
// then (with sparse layers) the K and V gradient accumulators,
// [B][n_kv][h_kv][head_dim] each, sized for 64-bit fixed point so that one
// workspace serves both backward entry points (fp32 sums use the first
// half), and the fixed-point bounds and scales (16 floats).
struct BwdLayout {
  size_t delta = 0, kt = 0, kt_bytes = 0, acc_k = 0, acc_v = 0, acc_elems = 0, total = 0;
  size_t bounds = 0;
  size_t qt = 0, dot = 0, rst = 0, rows_tiles = 0;
};

BwdLayout bwd_layout(const hs2_problem& p, int n_sparse) {
  BwdLayout L;
  size_t off = 0;
  L.delta = off;
  off += align_up((size_t)p.batch * p.h_q * p.n_q * sizeof(float));
  if (hs2::bwd_dq_uses_bf16_kernel(shape_of(p))) {
    L.kt = off;
    L.kt_bytes = (size_t)p.batch * p.h_kv * hs2::vt_keys_for(p.n_kv) * p.head_dim * 2;
    off += align_up(L.kt_bytes);
    L.rows_tiles = hs2::bwd_rows_layout_tiles(shape_of(p));
    const size_t tile_bytes = (size_t)64 * p.head_dim * 2;
    L.qt = off;
    off += align_up(L.rows_tiles * tile_bytes);
    L.dot = off;
    off += align_up(L.rows_tiles * tile_bytes);
    L.rst = off;
    off += align_up(L.rows_tiles * 128 * sizeof(float));
  }
  if (n_sparse > 0) {
    L.acc_elems = (size_t)p.batch * p.n_kv * p.h_kv * p.head_dim;
    L.acc_k = off;
    off += align_up(L.acc_elems * sizeof(long long));
    L.acc_v = off;
    off += align_up(L.acc_elems * sizeof(long long));
    L.bounds = off;
    off += align_up(16 * sizeof(float));
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

hs2_status hs2_backward_workspace_size(const hs2_problem* p, int32_t n_sparse_layers,
                                       size_t* bytes) {
  g_err.clear();
  HS2_TRY(check_problem(p));
  if (n_sparse_layers < 0) return fail(HS2_ERR_SHAPE, "n_sparse_layers %d", n_sparse_layers);
  if (!bytes) return fail(HS2_ERR_NULL, "bytes is NULL");
  *bytes = bwd_layout(*p, n_sparse_layers).total;
  return HS2_OK;
}

}  // extern "C"

namespace {

// Both backward entry points: `fixed` selects the sparse layers' 64-bit
// fixed-point K/V sums (deterministic) over fp32 atomics.
hs2_status block_backward(const hs2_problem* p, int32_t n_sparse_layers, const void* q_full,
                          const void* q_sparse, const void* k, const void* v,
                          const void* o_full, const void* o_sparse, const float* lse,
                          const int32_t* idx, const void* do_full, const void* do_sparse,
                          void* dq_full, void* dq_sparse, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream, bool fixed) {
  g_err.clear();
  HS2_TRY(check_problem(p));
  if (n_sparse_layers < 0) return fail(HS2_ERR_SHAPE, "n_sparse_layers %d", n_sparse_layers);
  HS2_TRY(check_ptr(q_full, "q_full"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  HS2_TRY(check_ptr(o_full, "o_full"));
  HS2_TRY(check_ptr(lse, "lse"));
  HS2_TRY(check_ptr(do_full, "do_full"));
  HS2_TRY(check_ptr(dq_full, "dq_full"));
  HS2_TRY(check_ptr(dk, "dk"));
  HS2_TRY(check_ptr(dv, "dv"));
  const bool sparse = n_sparse_layers > 0;
  HS2_TRY(check_ptr(q_sparse, "q_sparse", sparse));
  HS2_TRY(check_ptr(o_sparse, "o_sparse", sparse));
  HS2_TRY(check_ptr(idx, "idx", sparse));
  HS2_TRY(check_ptr(do_sparse, "do_sparse", sparse));
  HS2_TRY(check_ptr(dq_sparse, "dq_sparse", sparse));
  const BwdLayout L = bwd_layout(*p, n_sparse_layers);
  if (!workspace) return fail(HS2_ERR_NULL, "workspace is NULL (needs %zu bytes)", L.total);
  if (!aligned16(workspace)) return fail(HS2_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(HS2_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, L.total);

  const hipStream_t st = (hipStream_t)stream;
  const float scale_log2 = p->softmax_scale * 1.4426950408889634f;
  void* acc_k = sparse ? (char*)workspace + L.acc_k : nullptr;
  void* acc_v = sparse ? (char*)workspace + L.acc_v : nullptr;
  float* bounds = sparse ? fptr(workspace, L.bounds) : nullptr;   // 4 maxima, then 4 scales
  hs2::BwdPlan bp;
  bp.s = shape_of(*p);
  bp.scale = p->softmax_scale;
  bp.q = q_full; bp.k = k; bp.v = v; bp.o = o_full; bp.dout = do_full;
  bp.lse = lse; bp.delta = fptr(workspace, L.delta);
  bp.acc_k = acc_k; bp.acc_v = acc_v;
  bp.acc_fixed = sparse && fixed; bp.acc_scale = sparse ? bounds + 4 : nullptr;
  bp.dq = dq_full; bp.dk = dk; bp.dv = dv;
  {
    PassTimer t(st, HS2_PASS_BWD_PREP);
    HIP_TRY(hs2::launch_bwd_delta(bp, st), "backward Delta");
    if (L.kt_bytes) {
      // K in the tile-major transposed layout of the dQ kernel's K^T operand
      hs2::FwdPlan tp;
      tp.s = shape_of(*p);
      tp.v = k;
      tp.vt = (char*)workspace + L.kt;
      tp.vt_keys = hs2::vt_keys_for(p->n_kv);
      HIP_TRY(hs2::launch_v_transpose(tp, st), "K transpose");
      bp.kt = tp.vt;
      // Q and dO in the dK/dV kernel's transposed tile layout
      bp.qt = (char*)workspace + L.qt;
      bp.dot = (char*)workspace + L.dot;
      bp.rst = fptr(workspace, L.rst);
      HIP_TRY(hs2::launch_bwd_rows_layout(bp, st), "row layout");
    }
    if (sparse) {
      const size_t words = fixed ? 2 * L.acc_elems : L.acc_elems;
      HIP_TRY(hs2::launch_zero_f32(static_cast<float*>(acc_k), words, st), "zero accumulators");
      HIP_TRY(hs2::launch_zero_f32(static_cast<float*>(acc_v), words, st), "zero accumulators");
      if (fixed) {
        // fixed-point scales of the accumulators, from every sparse layer
        HIP_TRY(hs2::launch_zero_f32(bounds, 16, st), "zero bounds");
        hs2::SparseBwdBoundPlan bb;
        bb.q = q_sparse; bb.dout = do_sparse; bb.v = v;
        bb.q_rows = (size_t)n_sparse_layers * p->batch * p->n_q * p->h_q;
        bb.v_rows = (size_t)p->batch * p->n_kv * p->h_kv;
        bb.head_dim = p->head_dim;
        bb.bf16 = p->dtype == HS2_BF16;
        bb.rows = (double)n_sparse_layers * p->n_q * (p->h_q / p->h_kv);
        bb.scale = p->softmax_scale;
        bb.maxima = reinterpret_cast<unsigned*>(bounds);
        bb.scales = bounds + 4;
        HIP_TRY(hs2::launch_sparse_bwd_bounds(bb, st), "accumulator bounds");
      }
    }
  }
  if (sparse) {
    PassTimer t(st, HS2_PASS_BWD_SPARSE);
    const int G = p->h_q / p->h_kv;
    const int per = std::max(1, 64 / G);                     // layers per launch
    const size_t esz = p->dtype == HS2_BF16 ? 2 : 4;
    const size_t layer_bytes = (size_t)p->batch * p->n_q * p->h_q * p->head_dim * esz;
    for (int l0 = 0; l0 < n_sparse_layers; l0 += per) {
      hs2::SparseBwdPlan sp;
      sp.layers = std::min(per, n_sparse_layers - l0);
      sp.q = (const char*)q_sparse + l0 * layer_bytes;
      sp.o = (const char*)o_sparse + l0 * layer_bytes;
      sp.dout = (const char*)do_sparse + l0 * layer_bytes;
      sp.dq = (char*)dq_sparse + l0 * layer_bytes;
      sp.k = k; sp.v = v; sp.idx = idx; sp.acc_k = acc_k; sp.acc_v = acc_v;
      sp.fixed = fixed; sp.acc_scale = bounds + 4;
      sp.batch = p->batch; sp.n_q = p->n_q; sp.n_kv = p->n_kv; sp.h_q = p->h_q;
      sp.h_kv = p->h_kv; sp.head_dim = p->head_dim; sp.width = index_width(*p);
      sp.scale = p->softmax_scale; sp.scale_log2 = scale_log2;
      sp.bf16 = p->dtype == HS2_BF16;
      HIP_TRY(hs2::launch_sparse_bwd(sp, st), "sparse backward");
    }
  }
  {
    PassTimer t(st, HS2_PASS_BWD_DKDV);
    HIP_TRY(hs2::launch_bwd_dkdv(bp, st), "full-layer dK/dV");
  }
  {
    PassTimer t(st, HS2_PASS_BWD_DQ);
    HIP_TRY(hs2::launch_bwd_dq(bp, st), "full-layer dQ");
  }
  return HS2_OK;
}

}  // namespace

extern "C" {

hs2_status hs2_block_backward(const hs2_problem* p, int32_t n_sparse_layers, const void* q_full,
                              const void* q_sparse, const void* k, const void* v,
                              const void* o_full, const void* o_sparse, const float* lse,
                              const int32_t* idx, const void* do_full, const void* do_sparse,
                              void* dq_full, void* dq_sparse, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return block_backward(p, n_sparse_layers, q_full, q_sparse, k, v, o_full, o_sparse, lse, idx,
                        do_full, do_sparse, dq_full, dq_sparse, dk, dv, workspace,
                        workspace_bytes, stream, false);
}

hs2_status hs2_block_backward_deterministic(
    const hs2_problem* p, int32_t n_sparse_layers, const void* q_full, const void* q_sparse,
    const void* k, const void* v, const void* o_full, const void* o_sparse, const float* lse,
    const int32_t* idx, const void* do_full, const void* do_sparse, void* dq_full,
    void* dq_sparse, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return block_backward(p, n_sparse_layers, q_full, q_sparse, k, v, o_full, o_sparse, lse, idx,
                        do_full, do_sparse, dq_full, dq_sparse, dk, dv, workspace,
                        workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

// Workspace of a variable-length batch on the bf16 / head_dim 128 path:
// every prefill-shaped sequence (two or more queries) shares one full-
// attention launch, so their statistics (one 3 x h_q x n_q block per
// sequence, at 3 * h_q * cu_q[b]) and transposed V copies coexist; the
// score chunk (rows x the longest score row) follows. One-query sequences
// run afterwards on the decode path and reuse the workspace from the start.
struct VarlenLayout {
  size_t stats = 0, vt = 0, scores = 0;    // byte offsets
  size_t stride = 0;                       // floats per score row
  int chunk_rows = 0;
  int max_nq = 0;
  size_t min_bytes = 0, pref_bytes = 0;    // prefill part only
};

bool varlen_single_launch(const hs2_problem& p) {
  hs2::Shape s = shape_of(p);
  return hs2::prefill_uses_vt(s);
}

VarlenLayout varlen_layout(const hs2_problem& p, const int32_t* cu_q, const int32_t* cu_kv,
                           size_t ws_bytes) {
  VarlenLayout l;
  const size_t total_q = (size_t)cu_q[p.batch];
  size_t vt_tiles = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int nq = cu_q[b + 1] - cu_q[b], nkv = cu_kv[b + 1] - cu_kv[b];
    if (nq < 2) continue;
    hs2_problem pb = p;
    pb.batch = 1; pb.n_q = nq; pb.n_kv = nkv;
    l.stride = std::max(l.stride, score_stride(pb));
    l.max_nq = std::max(l.max_nq, nq);
    vt_tiles += (size_t)p.h_kv * (hs2::vt_keys_for(nkv) / 64);
  }
  if (l.max_nq == 0) return l;
  size_t off = 0;
  l.stats = off;
  off += align_up((size_t)3 * p.h_q * total_q * sizeof(float));
  l.vt = off;
  off += align_up(vt_tiles * 64 * p.head_dim * 2);
  l.scores = off;
  const size_t row_b = std::max<size_t>(l.stride, 1) * sizeof(float);
  l.min_bytes = off + align_up(row_b);
  size_t pref_rows = std::max<size_t>(128, CHUNK_TARGET / row_b / 128 * 128);
  pref_rows = std::min<size_t>(pref_rows, ((size_t)l.max_nq + 127) / 128 * 128);
  l.pref_bytes = off + align_up(pref_rows * row_b);
  if (ws_bytes != SIZE_MAX && ws_bytes >= l.min_bytes) {
    size_t rows = (ws_bytes - off) / row_b;
    if (rows >= 128) rows = rows / 128 * 128;
    rows = std::min<size_t>(rows, (size_t)l.max_nq);
    l.chunk_rows = (int)std::max<size_t>(rows, 1);
  }
  return l;
}

// Variable-length batches: sequence b owns queries cu_q[b] .. cu_q[b+1] and
// keys cu_kv[b] .. cu_kv[b+1] of the packed tensors. Checks the offsets and
// every non-empty sequence's problem (batch 1, its own n_q and n_kv), and
// returns the workspace the batch needs.
hs2_status check_varlen(const hs2_problem* p, const int32_t* cu_q, const int32_t* cu_kv,
                        size_t* min_bytes, size_t* pref_bytes, long long* total_q,
                        long long* total_kv) {
  if (!p) return fail(HS2_ERR_NULL, "problem is NULL");
  if (!cu_q || !cu_kv) return fail(HS2_ERR_NULL, "cu_seqlens arrays are NULL");
  if (p->batch < 1) return fail(HS2_ERR_SHAPE, "batch %d", p->batch);
  if (cu_q[0] != 0 || cu_kv[0] != 0) return fail(HS2_ERR_SHAPE, "cu_seqlens must start at 0");
  size_t mn = 0, pref = 0;
  for (int b = 0; b < p->batch; ++b) {
    const long long nq = (long long)cu_q[b + 1] - cu_q[b];
    const long long nkv = (long long)cu_kv[b + 1] - cu_kv[b];
    if (nq < 0 || nkv < 0)
      return fail(HS2_ERR_SHAPE, "cu_seqlens decrease at sequence %d", b);
    if (nq > nkv)
      return fail(HS2_ERR_SHAPE, "sequence %d: %lld queries > %lld keys", b, nq, nkv);
    if (nq == 0) continue;
    hs2_problem pb = *p;
    pb.batch = 1; pb.n_q = (int32_t)nq; pb.n_kv = (int32_t)nkv;
    HS2_TRY(check_problem(&pb));
    size_t m = 0, pr = 0;
    if (plan(pb, SIZE_MAX, nullptr, &m, &pr) != HS2_OK)
      return fail(HS2_ERR_SHAPE, "sequence %d: plan", b);
    mn = std::max(mn, m);
    pref = std::max(pref, pr);
  }
  if (varlen_single_launch(*p)) {
    // prefill-shaped sequences share the single-launch layout; one-query
    // sequences keep their own (decode) layout, reusing the same bytes
    size_t dmn = 0, dpref = 0;
    for (int b = 0; b < p->batch; ++b) {
      const int nq = cu_q[b + 1] - cu_q[b];
      if (nq != 1) continue;
      hs2_problem pb = *p;
      pb.batch = 1; pb.n_q = 1; pb.n_kv = cu_kv[b + 1] - cu_kv[b];
      size_t m = 0, pr = 0;
      plan(pb, SIZE_MAX, nullptr, &m, &pr);
      dmn = std::max(dmn, m);
      dpref = std::max(dpref, pr);
    }
    const VarlenLayout vl = varlen_layout(*p, cu_q, cu_kv, SIZE_MAX);
    mn = std::max(vl.min_bytes, dmn);
    pref = std::max(vl.pref_bytes, dpref);
  }
  if (min_bytes) *min_bytes = mn;
  if (pref_bytes) *pref_bytes = pref;
  if (total_q) *total_q = cu_q[p->batch];
  if (total_kv) *total_kv = cu_kv[p->batch];
  return HS2_OK;
}

}  // namespace

namespace {

// The prefill-shaped sequences of a bf16 / head_dim 128 variable-length
// batch: V transposes per sequence, one full-attention launch per group of
// up to VARLEN_MAX_SEQS sequences (all their row tiles fill the chip
// together), then per sequence the chunked score + selection and the
// sparse layers.
hs2_status run_varlen_prefill(const hs2_problem& p, int32_t n_sparse_layers,
                              const int32_t* cu_q, const int32_t* cu_kv, const void* q_full,
                              const void* q_sparse, const void* k, const void* v, void* o_full,
                              void* o_sparse, int32_t* idx, float* lse, void* ws, size_t ws_bytes,
                              size_t layer_elems, hipStream_t st) {
  const VarlenLayout vl = varlen_layout(p, cu_q, cu_kv, ws_bytes);
  if (vl.max_nq == 0) return HS2_OK;
  if (ws_bytes < vl.min_bytes) return fail(HS2_ERR_WORKSPACE, "workspace too small");
  const size_t esz = 2;
  const size_t qrow = (size_t)p.h_q * p.head_dim, krow = (size_t)p.h_kv * p.head_dim;
  const int width = index_width(p);
  const int G = p.h_q / p.h_kv;
  const int rows_per_tile = hs2::prefill_rows_per_tile();
  float* stats = fptr(ws, vl.stats);
  float* scores = fptr(ws, vl.scores);
  char* vt = (char*)ws + vl.vt;
  const bool block_mode = p.select == HS2_SELECT_BLOCK;
  auto sub = [&](int b) {
    hs2_problem pb = p;
    pb.batch = 1; pb.n_q = cu_q[b + 1] - cu_q[b]; pb.n_kv = cu_kv[b + 1] - cu_kv[b];
    return pb;
  };
  // V transposes, and the groups of the single launches
  std::vector<int> seqs;
  std::vector<int> vt0(p.batch, 0);
  int vt_tiles = 0;
  for (int b = 0; b < p.batch; ++b) {
    if (cu_q[b + 1] - cu_q[b] < 2) continue;
    const hs2_problem pb = sub(b);
    seqs.push_back(b);
    vt0[b] = vt_tiles;
    hs2::FwdPlan tf;
    tf.s = shape_of(pb);
    tf.v = (const char*)v + (size_t)cu_kv[b] * krow * esz;
    tf.vt = vt + (size_t)vt_tiles * 64 * p.head_dim * esz;
    tf.vt_keys = hs2::vt_keys_for(pb.n_kv);
    vt_tiles += p.h_kv * (tf.vt_keys / 64);
    PassTimer t(st, HS2_PASS_LAYOUT);
    HIP_TRY(hs2::launch_v_transpose(tf, st), "V transpose");
  }
  // longest context first: a row tile's work grows with its sequence's
  // key count, and the kernel hands out tiles in table order (every KV
  // head of a tile together), so the long tiles start first and the tail
  // is short
  std::vector<int> order = seqs;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return cu_kv[x + 1] - cu_kv[x] > cu_kv[y + 1] - cu_kv[y];
  });
  for (size_t g0 = 0; g0 < order.size(); g0 += hs2::VARLEN_MAX_SEQS) {
    hs2::VarlenSeqs d;
    d.n = (int)std::min<size_t>(hs2::VARLEN_MAX_SEQS, order.size() - g0);
    d.tile0[0] = 0;
    for (int s = 0; s < d.n; ++s) {
      const int b = order[g0 + s];
      d.q0[s] = cu_q[b];
      d.kv0[s] = cu_kv[b];
      d.nq[s] = cu_q[b + 1] - cu_q[b];
      d.nkv[s] = cu_kv[b + 1] - cu_kv[b];
      d.vt0[s] = vt0[b];
      d.tile0[s + 1] = d.tile0[s] + (d.nq[s] * G + rows_per_tile - 1) / rows_per_tile;
    }
    hs2::FwdPlan f;
    f.s = shape_of(p);
    f.q = q_full; f.k = k; f.v = v; f.o = o_full; f.stats = stats; f.lse = lse;
    f.vt = vt; f.vt_keys = 64;
    f.vl = &d;
    PassTimer t(st, HS2_PASS_FULL);
    HIP_TRY(hs2::launch_attn_fwd_prefill(f, st), "full attention (packed sequences)");
  }
  // per sequence: score chunks + selection, then the sparse layers
  for (int b : seqs) {
    const hs2_problem pb = sub(b);
    const hs2::Shape s1 = shape_of(pb);
    const char* qb = (const char*)q_full + (size_t)cu_q[b] * qrow * esz;
    const char* kb = (const char*)k + (size_t)cu_kv[b] * krow * esz;
    const char* vb = (const char*)v + (size_t)cu_kv[b] * krow * esz;
    int32_t* ib = idx + (size_t)cu_q[b] * width;
    float* sb = stats + (size_t)3 * p.h_q * cu_q[b];
    for (int q0 = 0; q0 < pb.n_q; q0 += vl.chunk_rows) {
      const int rows = std::min(vl.chunk_rows, pb.n_q - q0);
      hs2::ScorePlan sc;
      sc.s = s1; sc.b = 0; sc.q0 = q0; sc.rows = rows; sc.window = p.window;
      sc.q = qb; sc.k = kb; sc.stats = sb; sc.scores = scores; sc.score_stride = vl.stride;
      {
        PassTimer t(st, HS2_PASS_SCORE);
        HIP_TRY(hs2::launch_score_prefill(sc, st), "score");
      }
      hs2::SelectPlan sp;
      sp.rows = rows; sp.flat0 = q0; sp.n_q = pb.n_q; sp.n_kv = pb.n_kv;
      sp.top_k = p.top_k; sp.window = p.window; sp.width = width;
      sp.block_mode = block_mode; sp.block_size = p.block_size; sp.top_blocks = p.top_blocks;
      sp.scores = scores; sp.score_stride = vl.stride; sp.idx = ib;
      {
        PassTimer t(st, HS2_PASS_SELECT);
        HIP_TRY(hs2::launch_select(sp, st), "select");
      }
    }
    if (n_sparse_layers > 0)
      HS2_TRY(run_sparse(pb, n_sparse_layers, (const char*)q_sparse + (size_t)cu_q[b] * qrow * esz,
                         kb, vb, ib, (char*)o_sparse + (size_t)cu_q[b] * qrow * esz, st, nullptr,
                         layer_elems));
  }
  return HS2_OK;
}

// Sequence b of a packed batch on its own (batch 1, nq queries over nkv
// keys): the sequences no single full-attention launch covers. k, v point
// at the sequence's first key row, or at the pool when kv maps its rows
// through a page table; ws_bytes bytes of workspace from ws.
hs2_status run_sequence(const hs2_problem& p, int32_t n_sparse_layers, int b, int q0, int nq,
                        int nkv, const void* q_full, const void* q_sparse, const void* k,
                        const void* v, void* o_full, void* o_sparse, int32_t* idx, float* lse,
                        void* ws, size_t ws_bytes, size_t layer_elems, hipStream_t st,
                        const hs2::KvRows* kv) {
  const size_t esz = p.dtype == HS2_BF16 ? 2 : 4;
  const size_t qrow = (size_t)p.h_q * p.head_dim;
  hs2_problem pb = p;
  pb.batch = 1; pb.n_q = nq; pb.n_kv = nkv;
  Layout L;
  if (plan(pb, ws_bytes, &L, nullptr, nullptr) != HS2_OK)
    return fail(HS2_ERR_WORKSPACE, "sequence %d: workspace too small", b);
  const char* qb = (const char*)q_full + q0 * qrow * esz;
  char* ob = (char*)o_full + q0 * qrow * esz;
  int32_t* ib = idx + (size_t)q0 * index_width(p);
  float* lb = lse ? lse + (size_t)q0 * p.h_q : nullptr;
  HS2_TRY(run_full(pb, qb, k, v, ob, ib, lb, nullptr, ws, L, st, nullptr, kv));
  if (n_sparse_layers == 0) return HS2_OK;
  return run_sparse(pb, n_sparse_layers, (const char*)q_sparse + q0 * qrow * esz, k, v, ib,
                    (char*)o_sparse + q0 * qrow * esz, st, kv, layer_elems);
}

// Chunked prefill over a paged pool: sequence b appends n_q(b) = cu_q[b+1]
// - cu_q[b] tokens after its lens[b] cached ones. cu_kv holds the packed
// offsets of the logical lengths lens[b] + n_q(b); cu_st those of the
// staging copies, which only sequences with two or more new tokens get.
// Workspace: K staging, V staging (stage_bytes each), then what the
// variable-length batch of the same lengths needs.
struct PagedPlan {
  std::vector<int32_t> cu_kv, cu_st;
  size_t stage_bytes = 0;
  size_t min_bytes = 0, pref_bytes = 0;
  long long total_q = 0;
};

hs2_status plan_paged(const hs2_problem* p, const hs2_kv_pages* pages, const int32_t* cu_q,
                      const int32_t* lens, PagedPlan* pp, hs2::KvRows* kv) {
  if (!p) return fail(HS2_ERR_NULL, "problem is NULL");
  {
    hs2_problem p1 = *p;
    p1.n_q = 1;
    HS2_TRY(check_problem(&p1));
  }
  HS2_TRY(check_pages(*p, pages, kv));
  if (!cu_q || !lens) return fail(HS2_ERR_NULL, "cu_q or lens is NULL");
  if (cu_q[0] != 0) return fail(HS2_ERR_SHAPE, "cu_q must start at 0");
  pp->cu_kv.assign(p->batch + 1, 0);
  pp->cu_st.assign(p->batch + 1, 0);
  long long kv_sum = 0, st_sum = 0;
  for (int b = 0; b < p->batch; ++b) {
    const long long nq = (long long)cu_q[b + 1] - cu_q[b];
    if (nq < 0) return fail(HS2_ERR_SHAPE, "cu_q decreases at sequence %d", b);
    if (lens[b] < 0 || lens[b] + nq > p->n_kv)
      return fail(HS2_ERR_SHAPE, "sequence %d: %d cached + %lld new tokens exceed the capacity %d",
                  b, lens[b], nq, p->n_kv);
    kv_sum += lens[b] + nq;
    if (nq >= 2) st_sum += lens[b] + nq;
    if (kv_sum > INT32_MAX) return fail(HS2_ERR_UNSUPPORTED, "%lld tokens in the batch", kv_sum);
    pp->cu_kv[b + 1] = (int32_t)kv_sum;
    pp->cu_st[b + 1] = (int32_t)st_sum;
  }
  size_t mn = 0, pref = 0;
  HS2_TRY(check_varlen(p, cu_q, pp->cu_kv.data(), &mn, &pref, &pp->total_q, nullptr));
  const size_t row_bytes = (size_t)p->h_kv * p->head_dim * (p->dtype == HS2_BF16 ? 2 : 4);
  pp->stage_bytes = align_up((size_t)st_sum * row_bytes);
  pp->min_bytes = 2 * pp->stage_bytes + mn;
  pp->pref_bytes = 2 * pp->stage_bytes + pref;
  return HS2_OK;
}

}  // namespace

extern "C" {

hs2_status hs2_workspace_size_varlen(const hs2_problem* p, const int32_t* cu_q,
                                     const int32_t* cu_kv, size_t* min_bytes,
                                     size_t* preferred_bytes) {
  g_err.clear();
  if (!min_bytes && !preferred_bytes) return fail(HS2_ERR_NULL, "no output pointer");
  return check_varlen(p, cu_q, cu_kv, min_bytes, preferred_bytes, nullptr, nullptr);
}

hs2_status hs2_block_forward_varlen(const hs2_problem* p, int32_t n_sparse_layers,
                                    const int32_t* cu_q, const int32_t* cu_kv, const void* q_full,
                                    const void* q_sparse, const void* k, const void* v,
                                    void* o_full, void* o_sparse, int32_t* idx, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  size_t mn = 0;
  long long total_q = 0, total_kv = 0;
  HS2_TRY(check_varlen(p, cu_q, cu_kv, &mn, nullptr, &total_q, &total_kv));
  if (n_sparse_layers < 0) return fail(HS2_ERR_SHAPE, "n_sparse_layers %d", n_sparse_layers);
  HS2_TRY(check_ptr(q_full, "q_full"));
  HS2_TRY(check_ptr(k, "k"));
  HS2_TRY(check_ptr(v, "v"));
  HS2_TRY(check_ptr(o_full, "o_full"));
  HS2_TRY(check_ptr(idx, "idx"));
  HS2_TRY(check_ptr(lse, "lse", false));
  HS2_TRY(check_ptr(q_sparse, "q_sparse", n_sparse_layers > 0));
  HS2_TRY(check_ptr(o_sparse, "o_sparse", n_sparse_layers > 0));
  if (total_q > 0) {
    if (!workspace) return fail(HS2_ERR_NULL, "workspace is NULL (needs %zu bytes)", mn);
    if (!aligned16(workspace)) return fail(HS2_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < mn)
      return fail(HS2_ERR_WORKSPACE, "workspace %zu bytes < minimum %zu", workspace_bytes, mn);
  }
  const hipStream_t st = (hipStream_t)stream;
  const size_t esz = p->dtype == HS2_BF16 ? 2 : 4;
  const size_t krow = (size_t)p->h_kv * p->head_dim;          // elements per key token
  const size_t layer_elems = (size_t)total_q * p->h_q * p->head_dim;
  const bool single = varlen_single_launch(*p);
  if (single)
    HS2_TRY(run_varlen_prefill(*p, n_sparse_layers, cu_q, cu_kv, q_full, q_sparse, k, v, o_full,
                               o_sparse, idx, lse, workspace, workspace_bytes, layer_elems, st));
  for (int b = 0; b < p->batch; ++b) {
    const int q0 = cu_q[b], nq = cu_q[b + 1] - cu_q[b];
    if (nq == 0 || (single && nq >= 2)) continue;           // done in the single launch
    const int k0 = cu_kv[b];
    HS2_TRY(run_sequence(*p, n_sparse_layers, b, q0, nq, cu_kv[b + 1] - k0, q_full, q_sparse,
                         (const char*)k + k0 * krow * esz, (const char*)v + k0 * krow * esz,
                         o_full, o_sparse, idx, lse, workspace, workspace_bytes, layer_elems, st,
                         nullptr));
  }
  return HS2_OK;
}

hs2_status hs2_workspace_size_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                   const int32_t* cu_q, const int32_t* lens, size_t* min_bytes,
                                   size_t* preferred_bytes) {
  g_err.clear();
  if (!min_bytes && !preferred_bytes) return fail(HS2_ERR_NULL, "no output pointer");
  PagedPlan pp;
  hs2::KvRows kv;
  HS2_TRY(plan_paged(p, pages, cu_q, lens, &pp, &kv));
  if (min_bytes) *min_bytes = pp.min_bytes;
  if (preferred_bytes) *preferred_bytes = pp.pref_bytes;
  return HS2_OK;
}

hs2_status hs2_block_forward_paged(const hs2_problem* p, const hs2_kv_pages* pages,
                                   int32_t n_sparse_layers, const int32_t* cu_q,
                                   const int32_t* lens, const void* q_full, const void* q_sparse,
                                   const void* k_new, const void* v_new, void* k_pool,
                                   void* v_pool, void* o_full, void* o_sparse, int32_t* idx,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_err.clear();
  PagedPlan pp;
  hs2::KvRows kv;
  HS2_TRY(plan_paged(p, pages, cu_q, lens, &pp, &kv));
  if (n_sparse_layers < 0) return fail(HS2_ERR_SHAPE, "n_sparse_layers %d", n_sparse_layers);
  HS2_TRY(check_ptr(q_full, "q_full"));
  HS2_TRY(check_ptr(k_new, "k_new"));
  HS2_TRY(check_ptr(v_new, "v_new"));
  HS2_TRY(check_ptr(k_pool, "k_pool"));
  HS2_TRY(check_ptr(v_pool, "v_pool"));
  HS2_TRY(check_ptr(o_full, "o_full"));
  HS2_TRY(check_ptr(idx, "idx"));
  HS2_TRY(check_ptr(lse, "lse", false));
  HS2_TRY(check_ptr(q_sparse, "q_sparse", n_sparse_layers > 0));
  HS2_TRY(check_ptr(o_sparse, "o_sparse", n_sparse_layers > 0));
  if (pp.total_q == 0) return HS2_OK;
  if (!workspace) return fail(HS2_ERR_NULL, "workspace is NULL (needs %zu bytes)", pp.min_bytes);
  if (!aligned16(workspace)) return fail(HS2_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < pp.min_bytes)
    return fail(HS2_ERR_WORKSPACE, "workspace %zu bytes < minimum %zu", workspace_bytes,
                pp.min_bytes);
  const hipStream_t st = (hipStream_t)stream;
  const size_t row_bytes = (size_t)p->h_kv * p->head_dim * (p->dtype == HS2_BF16 ? 2 : 4);
  char* k_st = (char*)workspace;
  char* v_st = k_st + pp.stage_bytes;
  void* rest = v_st + pp.stage_bytes;
  const size_t rest_bytes = workspace_bytes - 2 * pp.stage_bytes;
  const int32_t* cu_st = pp.cu_st.data();

  // the new rows into their pages, and the prefill-shaped sequences' rows
  // into the staging buffers, up to STAGE_MAX_SEQS sequences per launch
  {
    PassTimer t(st, HS2_PASS_KV_STAGE);
    hs2::StageSeqs g;
    g.blk0[0] = 0;
    for (int b = 0; b <= p->batch; ++b) {
      if (b < p->batch) {
        const int nq = cu_q[b + 1] - cu_q[b];
        if (nq == 0) continue;
        const int r0 = nq >= 2 ? 0 : lens[b], end = lens[b] + nq;
        g.b[g.n] = b; g.r0[g.n] = r0; g.end[g.n] = end; g.lens[g.n] = lens[b];
        g.q0[g.n] = cu_q[b];
        g.st0[g.n] = nq >= 2 ? cu_st[b] : -1;
        g.blk0[g.n + 1] = g.blk0[g.n] + (end - r0 + hs2::STAGE_ROWS - 1) / hs2::STAGE_ROWS;
        ++g.n;
      }
      if (g.n == hs2::STAGE_MAX_SEQS || (b == p->batch && g.n > 0)) {
        HIP_TRY(hs2::launch_kv_stage(g, k_new, v_new, k_pool, v_pool, k_st, v_st, kv,
                                     (int)row_bytes, st),
                "KV append and staging");
        g.n = 0;
      }
    }
  }
  const size_t layer_elems = (size_t)pp.total_q * p->h_q * p->head_dim;
  // prefill-shaped sequences read their staged rows
  if (varlen_single_launch(*p)) {
    HS2_TRY(run_varlen_prefill(*p, n_sparse_layers, cu_q, cu_st, q_full, q_sparse, k_st, v_st,
                               o_full, o_sparse, idx, lse, rest, rest_bytes, layer_elems, st));
  } else {
    for (int b = 0; b < p->batch; ++b) {
      const int nq = cu_q[b + 1] - cu_q[b];
      if (nq < 2) continue;
      HS2_TRY(run_sequence(*p, n_sparse_layers, b, cu_q[b], nq, lens[b] + nq, q_full, q_sparse,
                           k_st + (size_t)cu_st[b] * row_bytes, v_st + (size_t)cu_st[b] * row_bytes,
                           o_full, o_sparse, idx, lse, rest, rest_bytes, layer_elems, st,
                           nullptr));
    }
  }
  // one-token sequences read the pool in place through their page-table row
  for (int b = 0; b < p->batch; ++b) {
    if (cu_q[b + 1] - cu_q[b] != 1) continue;
    hs2::KvRows kvb = kv;
    kvb.table = kv.table + (size_t)b * kv.max_pages;
    HS2_TRY(run_sequence(*p, n_sparse_layers, b, cu_q[b], 1, lens[b] + 1, q_full, q_sparse,
                         k_pool, v_pool, o_full, o_sparse, idx, lse, rest, rest_bytes, layer_elems,
                         st, &kvb));
  }
  return HS2_OK;
}

hs2_status hs2_profile_enable(int32_t on) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    for (auto& t : g_prof) {
      (void)hipEventDestroy(t.start);
      (void)hipEventDestroy(t.stop);
    }
    g_prof.clear();
  }
  g_prof_on = on != 0;
  return HS2_OK;
}

hs2_status hs2_profile_read(double* ms, int64_t* launches) {
  g_err.clear();
  if (!ms || !launches) return fail(HS2_ERR_NULL, "output arrays are NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int i = 0; i < HS2_N_PASSES; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  hs2_status st = HS2_OK;
  for (auto& t : g_prof) {
    float e = 0.f;
    hipError_t err = hipEventSynchronize(t.stop);
    if (err == hipSuccess) err = hipEventElapsedTime(&e, t.start, t.stop);
    if (err != hipSuccess && st == HS2_OK) st = device_fail(err, "profile events");
    ms[t.pass] += e;
    launches[t.pass] += 1;
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_prof.clear();
  return st;
}

const char* hs2_status_string(hs2_status s) {
  switch (s) {
    case HS2_OK: return "ok";
    case HS2_ERR_NULL: return "null pointer";
    case HS2_ERR_SHAPE: return "invalid shape";
    case HS2_ERR_UNSUPPORTED: return "unsupported";
    case HS2_ERR_WORKSPACE: return "workspace too small";
    case HS2_ERR_ALIGN: return "misaligned pointer";
    case HS2_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* hs2_last_error(void) { return g_err.c_str(); }

}  // extern "C"
