// Pass 2 of the full layer, specialised for bf16 and head dim 128: the
// head-summed softmax probability S(p, j) = sum_h 2^(t_h - m2_h) / l_h over
// every query head (same contract as score.hip; HySparse2 pages: openai-hub.net,
// section "From Hybrid SWA to HySparse2": the full layer decides which tokens
// matter).
//
// A work-group owns a 128-query x 256-key block of S and loops over every
// head in a fixed order (no atomics, bit-reproducible). Eight waves each
// hold a 64 x 64 block of S in registers and the K rows of their 64 keys
// for the G heads of the current KV head. Per head, the Q tile (32 KB) and
// the pass-1 statistics (m2, 1/l) of the 128 queries are loaded straight
// into LDS (global_load_lds), double-buffered; the next KV head's K rows
// (64 KB) are staged in LDS the same way while the current one is in use,
// and with two or more query heads per KV head the last query head of each
// KV head reads them into registers, each key block right after its last
// MFMAs, so a new KV head starts without a barrier or a wait of its own
// (0.5-1.5 % faster than reading them at its start).
// Chunks are XOR-swizzled so the MFMA operand reads are conflict-free; no
// global load in the loop writes a register, so nothing waits on the
// prefetches until the end of each head, and each load is a uniform
// per-head base plus a lane offset computed once per tile. Each probability costs one FMA
// (logit * c - m2), one exp2 and one FMA into the running sum. With a
// segment offset the kernel also writes, after each row's scores, the
// maximum of S over the candidate keys of every 64-key segment (one per
// wave and row), which the selection uses to read only the segments that
// can hold a selected key.
//
// Work-groups are ordered in blocks of 32 key tiles x all query tiles of
// the chunk, so a K tile is reused by every query tile from cache, and
// consecutive blocks land on the same XCD (shared L2).
#include "hs2_device.h"
#include "hs2_launch.h"

#include <type_traits>

namespace hs2 {

namespace {

constexpr int D = 128;
constexpr int TQ = 128;
constexpr int TKEY = 256;
constexpr int QT_BYTES = TQ * D * 2;          // 32 KB
constexpr int ST_BYTES = 2 * TQ * 4;          // m2 and 1/l of the tile's queries
constexpr int KT_BYTES = TKEY * D * 2;        // 64 KB: K rows of one KV head
// LDS: the two Q stages, the two statistics stages, the K buffer
constexpr int ST_BASE = 2 * QT_BYTES;
constexpr int K_BASE = ST_BASE + 2 * ST_BYTES;
constexpr int SMEM_BYTES = K_BASE + KT_BYTES;
constexpr int KT_BLOCK = 32;                  // key tiles per scheduling block

typedef __attribute__((address_space(3))) void lds_void;

// Q and K rows are 256 B (16 chunks). A 16-byte read of 64 lanes is served
// 32 lanes at a time from 128 banks (512 B), so rows of equal parity share
// banks; with bits 0 and 2 of the row's low four bits swapped in the
// swizzle, the 32 chunks a half wave reads (lane groups 0-1 or 2-3, one row
// per l16) land on distinct bank groups (the plain low four bits put chunks
// 4 grp + u and 4 (grp + 1) + u of rows l16 and l16 ^ 4 on the same banks).
__device__ __forceinline__ int row_swz(int row) { return (row & 10) | ((row & 1) << 2) | ((row >> 2) & 1); }
__device__ __forceinline__ int qswz(int row) { return row_swz(row); }
__device__ __forceinline__ int kswz(int row) { return row_swz(row); }

struct Score2Args {
  const __bf16* q; const __bf16* k;
  const float* stats;
  float* scores; size_t stride;
  int B, n_q, n_kv, h_q, h_kv;
  int b, q0, rows, window;
  int n_qt, n_kt;
  int swizzle;          // 0: ids in launch order (launches that are mostly causal triangle)
  float c;
  size_t seg_off;       // segment maxima offset within a row, 0 = do not write them
};

}  // namespace

// EARLY (G >= 2): each KV head's last query head reads the next K rows;
// otherwise each head reads its own K rows behind a barrier of its own.
template <bool EARLY>
__global__ __launch_bounds__(512, 2) void score_bf16_kernel(Score2Args a) {
  using OP = Op<__bf16, D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS targets stay scalar
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int wq = wave >> 2, wk = wave & 3;
  const int G = a.h_q / a.h_kv;
  const int q_off = a.n_kv - a.n_q;

  // blocked order: [key-tile block][query tile][key tile in block]
  const uint32_t lid = a.swizzle ? xcd_swizzle(blockIdx.x, gridDim.x) : blockIdx.x;
  const int per_block = a.n_qt * KT_BLOCK;
  const int kblk = lid / per_block;
  const int rem = lid - kblk * per_block;
  const int kts = min(KT_BLOCK, a.n_kt - kblk * KT_BLOCK);
  const int qt = rem / kts;
  const int kt = kblk * KT_BLOCK + (rem - qt * kts);

  const int r_lo = qt * TQ;
  const int r_hi = min(a.rows, r_lo + TQ) - 1;
  const int p_hi = q_off + a.q0 + r_hi;
  const int kj0 = kt * TKEY;
  if (kj0 > p_hi - a.window) return;                  // no candidate key here

  const __bf16* qseq = a.q + (size_t)a.b * a.n_q * a.h_q * D;
  const __bf16* kseq = a.k + (size_t)a.b * a.n_kv * a.h_kv * D;
  const size_t plane = (size_t)a.B * a.h_q * a.n_q;

  // The per-lane parts of the Q and statistics addresses (tile row, clamped
  // to the last row; 16-byte chunk) are the same for every head: a load is a
  // uniform per-head base plus a 32-bit lane offset computed once here.
  const int r_last = a.rows - 1 - r_lo;                 // last real row of the tile
  const __bf16* qtile = qseq + (size_t)(a.q0 + r_lo) * a.h_q * D;
  uint32_t q_lane[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int slot = (wave * 4 + t) * 64 + lane;
    const int r = slot >> 4, c = (slot & 15) ^ qswz(r);
    q_lane[t] = (uint32_t)(min(r, r_last) * a.h_q * D + c * 8) * 2;
  }
  // waves 0,1: m2 of rows 0..63, 64..127; waves 2,3: 1/l
  const float* st_tile = a.stats + ((wave >> 1) ? 2 : 0) * plane + (size_t)a.b * a.h_q * a.n_q + a.q0 + r_lo;
  const uint32_t st_lane = (uint32_t)min((wave & 1) * 64 + lane, r_last) * 4;
  auto issue = [&](int h, int stage) {
    char* base = smem + stage * QT_BYTES;
    const char* src = reinterpret_cast<const char*>(qtile + h * D);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(src + q_lane[t]), (lds_void*)(base + (wave * 4 + t) * 1024), 16, 0, 0);
    if (wave < 4)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(reinterpret_cast<const char*>(st_tile + (size_t)h * a.n_q) + st_lane),
                                       (lds_void*)(smem + ST_BASE + stage * ST_BYTES + wave * 256), 4, 0, 0);
  };

  // K rows of the tile's 256 keys for KV head g, into the K buffer
  // (the tile's key rows clamped to the last key, which no row reads back)
  auto issue_k = [&](int g) {
    char* base = smem + K_BASE;
    const char* src = reinterpret_cast<const char*>(kseq + ((size_t)kj0 * a.h_kv + g) * D);
    const int j_last = a.n_kv - 1 - kj0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int slot = (wave * 8 + t) * 64 + lane;
      const int r = slot >> 4, c = (slot & 15) ^ kswz(r);
      const uint32_t off = (uint32_t)(min(r, j_last) * a.h_kv * D + c * 8) * 2;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(src + off), (lds_void*)(base + (wave * 8 + t) * 1024), 16, 0, 0);
    }
  };

  f32x4 sacc[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Q rows wq * 64 + 16 qb + l16 all have the swizzle of l16 (it reads only
  // the row's low four bits), so query block qb sits a constant 16 rows (4 KB) past block 0 and
  // one offset per unit serves all four blocks; likewise the statistics
  const int srow0 = wq * 64 + l16;
  int qoff[4];                                        // [unit] byte offset in Q tile, block 0
#pragma unroll
  for (int u = 0; u < 4; ++u) qoff[u] = srow0 * 256 + (((4 * grp + u) ^ qswz(srow0)) << 4);

  issue(0, 0);
  issue_k(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // this KV head's K rows stay in registers for its G query heads
  bf16x8 kf[4][4];
  auto read_k = [&](int kb) __attribute__((always_inline)) {
    const int row = wk * 64 + kb * 16 + l16;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kf[kb][u] = *reinterpret_cast<const bf16x8*>(
          smem + K_BASE + row * 256 + (((4 * grp + u) ^ kswz(row)) << 4));
  };
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) read_k(kb);
  // With two or more query heads per KV head, the K buffer is refilled with
  // the next KV head's rows at the start of each KV head, and the last query
  // head of a KV head reads them into registers, each key block right after
  // its last MFMAs: no barrier of its own and no wait at the next KV head's
  // start (every wave's reads end before the head-end barrier, which also
  // covers the landing of the refill issued a head or more earlier). With
  // one query head per KV head, each head reads K at its start behind a
  // barrier of its own.
  constexpr bool early = EARLY;
  if constexpr (early) {
    __syncthreads();                                  // every wave holds K(0)
    if (a.h_kv > 1) issue_k(1);
  }

  // one query head; reload_c: read the next KV head's K rows on the way
  auto head = [&](int h, auto reload_c) __attribute__((always_inline)) {
    constexpr bool reload = decltype(reload_c)::value;
    const int stage = h & 1;
    if (h + 1 < a.h_q) issue(h + 1, stage ^ 1);
    const char* base = smem + stage * QT_BYTES;
    const float* st = reinterpret_cast<const float*>(smem + ST_BASE + stage * ST_BYTES);

    // Q fragments of query block qb + 1 are read while block qb computes.
    // The 16 (qb, kb) blocks form a software pipeline: the four MFMAs of
    // block b are interleaved one by one with the exp work of block b - 1,
    // so the matrix core and the VALU stay busy together.
    bf16x8 qf[2][4];
    float m2v[2], ilv[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) qf[0][u] = *reinterpret_cast<const bf16x8*>(base + qoff[u]);
    m2v[0] = st[srow0];
    ilv[0] = st[TQ + srow0];
    f32x4 xp = f32x4{0.f, 0.f, 0.f, 0.f};
    float pm2 = 0.f, pil = 0.f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int qb = b >> 2, kb = b & 3, cur = qb & 1;
      if (kb == 0 && qb + 1 < 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          qf[cur ^ 1][u] = *reinterpret_cast<const bf16x8*>(base + qoff[u] + (qb + 1) * 4096);
        m2v[cur ^ 1] = st[srow0 + (qb + 1) * 16];
        ilv[cur ^ 1] = st[TQ + srow0 + (qb + 1) * 16];
      }
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) x = OP::mma(kf[kb][u], qf[cur][u], x);
      // the last query block is the last use of key block kb
      if (reload && qb == 3) read_k(kb);
      if (b > 0) {
        const int pqb = (b - 1) >> 2, pkb = (b - 1) & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[pqb][pkb][e] = fmaf(fast_exp2(fmaf(xp[e], a.c, pm2)), pil, sacc[pqb][pkb][e]);
        // two MFMAs first: the previous block's logits leave its last MFMA
        // only about two MFMA issue slots after it
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      xp = x;
      pm2 = -m2v[cur];
      pil = ilv[cur];
      // hard fence: a block's own exp work may not move up next to its MFMAs
      // (it would wait out their latency); it runs with the next block
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sacc[3][3][e] = fmaf(fast_exp2(fmaf(xp[e], a.c, pm2)), pil, sacc[3][3][e]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if constexpr (!early) {
    for (int h = 0; h < a.h_q; ++h) {
      if (h > 0) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) read_k(kb);
      }
      __syncthreads();                                // every wave holds K(h)
      if (h + 1 < a.h_kv) issue_k(h + 1);
      head(h, std::false_type{});
    }
  } else {
    // KV heads with a successor: the last query head reads the next K rows
    for (int g = 0; g + 1 < a.h_kv; ++g) {
      if (g > 0) issue_k(g + 1);
      for (int hh = 0; hh + 1 < G; ++hh) head(g * G + hh, std::false_type{});
      head(g * G + G - 1, std::true_type{});
    }
    for (int h = (a.h_kv - 1) * G; h < a.h_q; ++h) head(h, std::false_type{});
  }

  // keys past n_kv (tile tail) are never read back: rows only use j <= p - w
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int r = r_lo + srow0 + qb * 16;
    if (r >= a.rows) continue;
    float* out = a.scores + (size_t)r * a.stride + kj0 + wk * 64 + 4 * grp;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<f32x4*>(out + kb * 16) = sacc[qb][kb];
  }
  // the wave's 64 keys are one segment: per query, the maximum of its
  // candidate keys there (the row's lanes l16 + 16 grp hold 16 keys each)
  if (a.seg_off) {
    const int s0 = kj0 + wk * 64;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int r = r_lo + srow0 + qb * 16;
      const int lim = q_off + a.q0 + r - a.window;    // last candidate key of row r
      float m = -1.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s0 + kb * 16 + 4 * grp + e <= lim) m = max2f(m, sacc[qb][kb][e]);
      m = row_group_max(m);
      if (grp == 0 && r < a.rows && s0 <= lim)
        a.scores[(size_t)r * a.stride + a.seg_off + (s0 >> 6)] = m;
    }
  }
}

bool score_uses_bf16_kernel(const Shape& s) { return s.bf16 && s.head_dim == D; }

hipError_t launch_score_prefill_generic(const ScorePlan& p, hipStream_t st);

hipError_t launch_score_prefill(const ScorePlan& p, hipStream_t st) {
  if (!score_uses_bf16_kernel(p.s)) return launch_score_prefill_generic(p, st);
  Score2Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.stats = p.stats; a.scores = p.scores; a.stride = p.score_stride;
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.b = p.b; a.q0 = p.q0; a.rows = p.rows; a.window = p.window; a.c = p.s.scale_log2;
  a.seg_off = p.seg_off;
  const int q_off = a.n_kv - a.n_q;
  const int n_cand_max = q_off + p.q0 + p.rows - p.window;
  if (n_cand_max <= 0) return hipSuccess;
  a.n_qt = (p.rows + TQ - 1) / TQ;
  a.n_kt = (n_cand_max + TKEY - 1) / TKEY;
  // When the chunk's first row has under half the candidates of its last
  // (the causal triangle dominates, as in a prefill from position 0), many
  // blocks exit at once, and ids in launch order ran 37 % faster at the 32K
  // prefill than the XCD swizzle; chunks deep in a long context (all rows
  // with nearly the same candidates) keep the swizzle.
  const int n_cand_min = q_off + p.q0 - p.window + 1;
  a.swizzle = 2 * n_cand_min >= n_cand_max ? 1 : 0;
  const dim3 grid((unsigned)((size_t)a.n_qt * a.n_kt));
  if (a.h_q / a.h_kv >= 2) {
    struct ScoreLdsTag {};
    const hipError_t e = ensure_dynamic_lds<ScoreLdsTag>((const void*)score_bf16_kernel<true>, SMEM_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(score_bf16_kernel<true>, grid, dim3(512), SMEM_BYTES, st, a);
  } else {
    struct ScoreLdsTag1 {};
    const hipError_t e = ensure_dynamic_lds<ScoreLdsTag1>((const void*)score_bf16_kernel<false>, SMEM_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(score_bf16_kernel<false>, grid, dim3(512), SMEM_BYTES, st, a);
  }
  return hipGetLastError();
}

}  // namespace hs2
