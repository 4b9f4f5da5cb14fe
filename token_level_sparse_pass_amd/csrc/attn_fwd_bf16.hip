// Pass 1 of the full layer, specialised for bf16 and head dim 128 (the
// long-context workloads). Same contract as attn_fwd.hip: causal GQA
// attention over the shared K/V plus per-(query, head) statistics
// (m2, l) and LSE.
//
// Differences from the generic kernel, all aimed at keeping the MFMA pipe
// fed with as few instructions around it as possible:
//  * V is transposed once per call into a tile-major copy in the workspace,
//    Vt[b][g][tile][d][64 keys], so the PV product reads its operands with
//    16-byte LDS loads instead of transposing in registers;
//  * K and Vt tiles go straight from global memory into LDS
//    (global_load_lds_dwordx4) through two-stage rings, with XOR-swizzled
//    16-byte chunks so the MFMA operand reads are free of bank conflicts;
//    the tile loop is unrolled by two so each stage's LDS offsets are
//    immediates of the read instructions, and tiles that need no causal
//    mask run a copy of the loop body without one; a load's global address
//    is a uniform tile base plus a lane offset computed once, and its LDS
//    target is uniform, so the loads cost almost no vector instructions;
//  * the eight waves form two groups half a tile apart (waves w and w + 4
//    share a SIMD): a tile step is an MFMA phase (the previous tile's PV
//    product, then this tile's logits) and a VALU phase (this tile's
//    softmax), and the groups pass the tile barrier at different points of
//    it, so one wave's MFMAs run beside its SIMD partner's softmax (1-2 %
//    faster than all eight waves in step; counters put both the MFMA and the
//    VALU pipe near half busy, so the loop is latency bound at two waves per
//    SIMD rather than bound by either pipe);
//  * row maxima use three-input max instructions and the gfx950 permlane
//    swaps (no LDS round trip for the cross-row step); this file is built
//    with -fno-honor-nans so that fmaxf does not first quiet every operand
//    (the kernel never sees a NaN: masked logits are -inf); each lane first
//    tests its own 16 logits of a row against the running max, and the
//    cross-lane step runs only on tiles where some lane would move it (a row
//    moves exactly when one of its lanes does: 1.5-2.5 % faster, same
//    results); that test compares the raw lane maximum with a threshold
//    (m + gap) / c kept beside the running max, so it costs one compare
//    (about 1 % faster; the exact test inside decides the move);
//  * the keys of a 64-key tile are assigned to MFMA rows in a permuted order
//    such that the P^T operand of each lane covers 8 consecutive keys;
//  * the running max is only moved (and O rescaled) when it grows by more
//    than 2^8, so the rescale multiply almost never runs; exponents are
//    formed with one FMA (logit * c - m) from the raw MFMA result;
//  * on open tiles after the first (every row then holds a finite running
//    max) the probabilities are formed with the max as it stands and no
//    lane maximum is taken: only where a lane's 16 probabilities sum past
//    2^12 is the max looked at again (from log2 of the largest probability,
//    or, when one overflowed fp32, from the tile's logits formed again with
//    K read from memory); the sums serve the row sums as well (2.5 % faster
//    at 262K and 1M);
//  * the causal mask is applied only on tiles that reach the diagonal.
// Rows, as in the generic kernel, are (query, head-of-group) pairs: RBW
// 16-row MFMA blocks per wave, eight waves (two per SIMD) per work-group,
// all sharing each tile in LDS. Each wave reads a whole K and V^T tile from
// LDS per 64 keys (512 B per MFMA); the LDS pipe is busy under half of its
// cycles.
#include "hs2_device.h"
#include "hs2_launch.h"

#include <type_traits>

namespace hs2 {

#ifndef FWD_WAVES
#define FWD_WAVES 8
#endif

namespace {

constexpr int TK = 64;              // keys per tile
constexpr int D = 128;
constexpr int KT_BYTES = TK * D * 2;        // 16 KB
constexpr int STAGE_BYTES = 2 * KT_BYTES;   // K tile + Vt tile
constexpr float RESCALE_GAP = 8.0f;         // log2 units
constexpr float SPEC_LIMIT = 4096.0f;       // a lane's tile row sum past this rechecks the max
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void;

// chunk swizzles: K tile rows are 256 B (16 chunks), Vt rows 128 B (8 chunks).
// A 16-byte read of 64 lanes is served 32 lanes at a time from 128 banks
// (512 B), so two rows of equal parity share banks: the K swizzle makes the
// 32 chunks that a half wave reads from 16 rows (lane groups 0-1 or 2-3,
// one row per l16) land on distinct bank groups. It is built from row bits
// 0, 1, 3 and 4 only (the bits l16 sets in tile_key), with row bits 0 and 3
// in swapped places: for fixed row parity, chunks 4 grp + u and
// 4 (grp + 1) + u then never meet (halves the LDS cycles of the K reads).
__device__ __forceinline__ int kswz(int row) {
  return ((row >> 3) & 1) | (row & 2) | ((row & 1) << 2) | (((row >> 4) & 1) << 3);
}
__device__ __forceinline__ int vswz(int row) { return (row >> 1) & 7; }

// key held in MFMA row m of key block kb: lane group q of the P^T operand
// then owns keys 32*(kb/2) + 8q .. +7 of the tile
__device__ __forceinline__ int tile_key(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct Fwd2Args {
  const __bf16* q; const __bf16* k; const __bf16* vt;
  __bf16* o; float* stats; float* lse;
  int B, n_q, n_kv, h_q, h_kv, n_rt, vt_tiles;
  float c;                           // softmax scale * log2(e)
  VarlenSeqs vl;                     // vl.n > 0: packed sequences, one launch
};

}  // namespace

// V [B][n_kv][h_kv][128] -> Vt [B][h_kv][tile][128][64], zero past n_kv.
__global__ __launch_bounds__(256) void transpose_v_kernel(const __bf16* v, __bf16* vt, int n_kv,
                                                          int h_kv, int vt_tiles) {
  __shared__ uint16_t tile[TK][D + 8];
  const int t = blockIdx.x % vt_tiles;
  const int bg = blockIdx.x / vt_tiles;
  const int g = bg % h_kv;
  const int b = bg / h_kv;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + ((size_t)b * n_kv * h_kv + g) * D;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int u = threadIdx.x + 256 * it;
    const int r = u >> 4, c = u & 15;
    const int j = t * TK + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j < n_kv) val = *reinterpret_cast<const uint4*>(src + (size_t)j * h_kv * D + c * 8);
    *reinterpret_cast<uint4*>(&tile[r][c * 8]) = val;
  }
  __syncthreads();
  uint16_t* dst = reinterpret_cast<uint16_t*>(vt) + (((size_t)b * h_kv + g) * vt_tiles + t) * D * TK;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int u = threadIdx.x + 256 * it;       // 1024 output chunks of 8 keys
    const int d = u >> 3, c = u & 7;
    uint16_t e[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) e[x] = tile[c * 8 + x][d];
    uint4 w;
    w.x = e[0] | ((uint32_t)e[1] << 16);
    w.y = e[2] | ((uint32_t)e[3] << 16);
    w.z = e[4] | ((uint32_t)e[5] << 16);
    w.w = e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<uint4*>(dst + (size_t)d * TK + c * 8) = w;
  }
}

// RBW 16-row blocks per wave, NWV waves per work-group (all of them share
// each K/V tile in LDS).
template <int RBW, int NWV>
__global__ __launch_bounds__(64 * NWV, 2) void attn_fwd_bf16_kernel(Fwd2Args a) {
  using OP = Op<__bf16, D>;
  constexpr int ROWS = 16 * RBW * NWV;                  // rows per work-group
  // a fixed-size array: its address is a constant, so stage and row offsets
  // fold into the immediates of the LDS instructions
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS targets stay scalar
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;

  // this work-group's sequence: its lengths, token offsets into the packed
  // tensors, transposed-V block, and its statistics block (3 planes of
  // h_q x n_q, as a batch-1 call lays them out)
  int g, rt, nq, nkv;
  size_t qtok0, ktok0, vt_tile0, st0, plane;
  int vt_tiles;
  if (a.vl.n > 0) {
    // KV head fastest, then the table's tiles in order (sequences longest
    // context first, each heaviest tile first), as the dispatcher starts
    // them: longest first over the whole grid
    g = (int)(blockIdx.x % a.h_kv);
    const int t = (int)(blockIdx.x / a.h_kv);
    int s = 0;
    while (s + 1 < a.vl.n && t >= a.vl.tile0[s + 1]) ++s;
    nq = a.vl.nq[s];
    nkv = a.vl.nkv[s];
    rt = a.vl.tile0[s + 1] - 1 - t;                     // heavy tiles first
    qtok0 = a.vl.q0[s];
    ktok0 = a.vl.kv0[s];
    vt_tiles = (nkv + TK - 1) / TK;
    vt_tile0 = (size_t)a.vl.vt0[s] + (size_t)g * vt_tiles;
    st0 = (size_t)3 * a.h_q * a.vl.q0[s];
    plane = (size_t)a.h_q * nq;
  } else {
    // longest first over the whole grid: row tile n_rt - 1 of every
    // (sequence, KV head), then n_rt - 2, ...; work-groups start in id
    // order on whichever CU frees up, so the long causal tiles start first
    // and the tail is short (heaviest first within each KV head, through
    // the XCD swizzle, ran 27 % longer at a 32K-token prefill)
    rt = a.n_rt - 1 - (int)(blockIdx.x / (a.B * a.h_kv));
    const int bg = blockIdx.x % (a.B * a.h_kv);
    const int b = bg % a.B;
    g = bg / a.B;
    nq = a.n_q;
    nkv = a.n_kv;
    qtok0 = (size_t)b * a.n_q;
    ktok0 = (size_t)b * a.n_kv;
    vt_tiles = a.vt_tiles;
    vt_tile0 = ((size_t)b * a.h_kv + g) * a.vt_tiles;
    st0 = (size_t)b * a.h_q * a.n_q;
    plane = (size_t)a.B * a.h_q * a.n_q;
  }
  (void)vt_tiles;
  const int R = nq * G;
  const int q_off = nkv - nq;
  const int r0 = rt * ROWS;
  const int i_hi = min(nq - 1, (r0 + ROWS - 1) / G);
  const int p_lo = q_off + r0 / G;                      // smallest position here
  const int p_hi = q_off + i_hi;
  const int n_tiles = (p_hi + TK) / TK;
  const int n_full = (p_lo + 1) / TK;                   // tiles with no masked key

  const size_t kstride = (size_t)a.h_kv * D;
  const __bf16* kseq = a.k + (ktok0 * a.h_kv + g) * D;
  const __bf16* vtseq = a.vt + vt_tile0 * (size_t)(D * TK);
  const __bf16* qseq = a.q + qtok0 * a.h_q * D;
  __bf16* oseq = a.o + qtok0 * a.h_q * D;
  float* stats = a.stats + st0;
  float* lse = a.lse ? a.lse + (a.vl.n > 0 ? (size_t)a.h_q * qtok0 : st0) : nullptr;

  // ---- Q fragments and row positions ----
  Frag<__bf16, D> qf[RBW];
  int row_pos[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * 16 * RBW + rb * 16 + l16;
    if (r < R) {
      const int i = r / G, hh = r - (r / G) * G;
      load_slice<__bf16, D>(qf[rb], qseq + ((size_t)i * a.h_q + g * G + hh) * D, lane);
      row_pos[rb] = q_off + i;
    } else {
      zero_slice<__bf16, D>(qf[rb]);
      row_pos[rb] = -1;
    }
  }

  // ---- two groups of four waves, half a tile apart ----
  // Waves w and w + 4 share a SIMD. Each wave's tile step is an MFMA phase
  // (the previous tile's PV product, then this tile's logits) followed by a
  // VALU phase (the softmax that forms this tile's P). The leading group
  // (waves 0-3) passes tile barrier t before its MFMA phase of tile t, the
  // other group between its MFMA and VALU phases of tile t - 1, so on every
  // SIMD one wave's MFMAs run beside the other wave's softmax arithmetic
  // instead of both waves reaching each phase together.
  // Tiles move through two-stage rings: right after barrier t every wave
  // issues its share of K(t + 1) (into the stage of K(t - 1), whose logits
  // both groups formed before barrier t) and of Vt(t) (into the stage of
  // Vt(t - 2), whose PV product both groups finished before barrier t); a
  // wave waits for its own loads before its next barrier, so both tiles are
  // in LDS for every wave after barrier t + 1, before either is read.
  const bool lead = wave < 4;
  static_assert(NWV == 8, "two groups of four waves");
  constexpr int CPT = 1024 / (64 * NWV);                // 16-byte chunks per thread per tensor

  // The chunks a lane moves sit at fixed byte offsets from the tile's start
  // (K row r of the tile, Vt row d), so a load is a uniform tile base plus a
  // per-lane 32-bit offset computed once here, and the LDS targets are
  // uniform: no per-tile vector address arithmetic. Only a tile that runs
  // past n_kv clamps its K rows (to row n_kv - 1, whose logits are masked).
  int k_row[CPT];
  uint32_t k_off[CPT], k_col[CPT], v_off[CPT];
#pragma unroll
  for (int t = 0; t < CPT; ++t) {
    const int slot = (wave * CPT + t) * 64 + lane;
    const int r = slot >> 4, c = (slot & 15) ^ kswz(r);
    k_row[t] = r;
    k_col[t] = (uint32_t)c * 16;
    k_off[t] = (uint32_t)((size_t)r * kstride * 2) + k_col[t];
    const int d = slot >> 3, cv = (slot & 7) ^ vswz(d);
    v_off[t] = (uint32_t)(d * TK + cv * 8) * 2;
  }
  auto issue_k = [&](int tile, int stage) __attribute__((always_inline)) {
    char* base = smem + stage * STAGE_BYTES;
    const int j0 = tile * TK;
    if (j0 + TK <= nkv) {
      const char* src = reinterpret_cast<const char*>(kseq + (size_t)j0 * kstride);
#pragma unroll
      for (int t = 0; t < CPT; ++t)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(src + k_off[t]), (lds_void*)(base + (wave * CPT + t) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int t = 0; t < CPT; ++t) {
        const int key = min(j0 + k_row[t], nkv - 1);
        const char* src = reinterpret_cast<const char*>(kseq + (size_t)key * kstride) + k_col[t];
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(src), (lds_void*)(base + (wave * CPT + t) * 1024), 16, 0, 0);
      }
    }
  };
  auto issue_v = [&](int tile, int stage) __attribute__((always_inline)) {
    char* base = smem + stage * STAGE_BYTES;
    const char* vsrc = reinterpret_cast<const char*>(vtseq + (size_t)tile * (D * TK));
#pragma unroll
    for (int t = 0; t < CPT; ++t)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const __bf16*>(vsrc + v_off[t]), (lds_void*)(base + KT_BYTES + (wave * CPT + t) * 1024), 16, 0, 0);
  };

  float m_run[RBW];
  float thr[RBW];                                       // (m_run + gap) / c: a raw logit past it moves the max
  float lsum[RBW];                                      // this lane's share of the tile's row sums
  float l_s[RBW], l_c[RBW];                             // compensated row sums
  f32x4 acc[RBW][8];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m_run[rb] = -1e30f;
    thr[rb] = -1e30f;
    l_s[rb] = 0.f;
    l_c[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS offsets that do not change between tiles. The K row of
  // key block kb held by lane (grp, l16) is tile_key(kb, l16), whose swizzle
  // kswz() does not depend on kb, so the block moves the row by a constant
  // (KB_OFF[kb], an immediate of the read); likewise the Vt row of head-dim
  // block db is db * 16 + l16, whose swizzle does not depend on db.
  int koff[4];                                          // [unit] byte offset, key block 0
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = tile_key(0, l16) * 256 + (((4 * grp + u) ^ kswz(tile_key(0, l16))) << 4);
  int voff[2];                                          // [step] byte offset, head-dim block 0
#pragma unroll
  for (int st = 0; st < 2; ++st) voff[st] = KT_BYTES + l16 * 128 + (((4 * st + grp) ^ vswz(l16)) << 4);

  f32x4 s[RBW][4];                                      // this tile's logits^T
  bf16x8 pu[RBW][2];                                    // the previous tile's P^T operands

  // O^T += V^T . P^T for the tile whose P is in pu (its Vt rows at vbase),
  // then the compensated add of that tile's row sums (formed with its
  // probabilities in the softmax phase)
  auto pv = [&](auto stage_c) __attribute__((always_inline)) {
    const char* vbase = smem + decltype(stage_c)::value * STAGE_BYTES;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(vbase + voff[0] + db * 2048);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(vbase + voff[1] + db * 2048);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        acc[rb][db] = OP::mma(v0, pu[rb][0], acc[rb][db]);
        acc[rb][db] = OP::mma(v1, pu[rb][1], acc[rb][db]);
      }
    }
    // compensated add of the tile's row sums (formed with its probabilities)
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const float y = lsum[rb] - l_c[rb];
      const float tt = l_s[rb] + y;
      l_c[rb] = (tt - l_s[rb]) - y;
      l_s[rb] = tt;
    }
  };
  // logits^T for 4 key blocks x 2 row blocks; the K fragments of block
  // kb + 1 are read from LDS while block kb's MFMAs run
  auto qk = [&](auto stage_c) __attribute__((always_inline)) {
    const char* kbase = smem + decltype(stage_c)::value * STAGE_BYTES;
    bf16x8 kf[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kf[0][u] = *reinterpret_cast<const bf16x8*>(kbase + koff[u]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < 4) {
        const int kb_off = (tile_key(kb + 1, 0) - tile_key(0, 0)) * 256;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kf[cur ^ 1][u] = *reinterpret_cast<const bf16x8*>(kbase + koff[u] + kb_off);
      }
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) x = OP::mma(kf[cur][u], qf[rb].u[u], x);
        s[rb][kb] = x;
      }
    }
  };
  // softmax of tile t: row maxima, lazy rescale, P = 2^(s c - m), row sums,
  // P^T operands in bf16
  // this lane's 16 probabilities of row block rb summed in key order
  // (starting from the first term: the probabilities are never -0, so
  // 0 + x = x and the sum is the one a zero start gives)
  auto row_part = [&](int rb) __attribute__((always_inline)) {
    float ls = s[rb][0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (kb + e > 0) ls += s[rb][kb][e];
    return ls;
  };
  // softmax of tile t: row maxima, lazy rescale, P = 2^(s c - m), row sums,
  // P^T operands in bf16. The exact form forms each lane's maximum first; the
  // speculative form (open tiles after the first, whose rows all hold a
  // finite running max) forms P with the running max as it stands and only
  // looks for a new maximum on the rare tiles where a lane's row sum passes
  // SPEC_LIMIT (then every P was at most that, or some logit ran past the
  // range of fp32 and the tile's logits are recomputed from K in memory)
  auto softmax = [&](int t, auto masked_c, auto spec_c) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_c)::value;
    constexpr bool spec = decltype(spec_c)::value;
    const int j0 = t * TK;
    // (a raised issue priority for this phase, s_setprio, had gained 0.5 %
    // before the speculative form; with the shorter phase it cost about 1 %)
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      if constexpr (spec) {
        const float neg_m = -m_run[rb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[rb][kb][e] = fast_exp2(fmaf(s[rb][kb][e], a.c, neg_m));
        float ls = row_part(rb);
        if (__builtin_amdgcn_ballot_w64(!(ls <= SPEC_LIMIT))) {
          // the lane's largest probability; +inf: a logit passed the running
          // max by more than fp32 holds, so the logits are formed again
          const float pmax = max2f(max3f(max3f(s[rb][0][0], s[rb][0][1], s[rb][0][2]),
                                         max3f(s[rb][0][3], s[rb][1][0], s[rb][1][1]),
                                         max3f(s[rb][1][2], s[rb][1][3], s[rb][2][0])),
                                   max3f(max3f(s[rb][2][1], s[rb][2][2], s[rb][2][3]),
                                         max3f(s[rb][3][0], s[rb][3][1], s[rb][3][2]), s[rb][3][3]));
          const bool lost = __builtin_amdgcn_ballot_w64(pmax == INFINITY) != 0;
          float m_tile;
          if (lost) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const __bf16* krow = kseq + (size_t)(j0 + tile_key(kb, l16)) * kstride + 8 * (4 * grp);
              f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int u = 0; u < 4; ++u)
                x = OP::mma(*reinterpret_cast<const bf16x8*>(krow + 8 * u), qf[rb].u[u], x);
              s[rb][kb] = x;
            }
            const float lmax = max2f(max3f(max3f(s[rb][0][0], s[rb][0][1], s[rb][0][2]),
                                           max3f(s[rb][0][3], s[rb][1][0], s[rb][1][1]),
                                           max3f(s[rb][1][2], s[rb][1][3], s[rb][2][0])),
                                     max3f(max3f(s[rb][2][1], s[rb][2][2], s[rb][2][3]),
                                           max3f(s[rb][3][0], s[rb][3][1], s[rb][3][2]), s[rb][3][3]));
            m_tile = row_group_max(lmax) * a.c;
          } else {
            m_tile = m_run[rb] + __builtin_amdgcn_logf(row_group_max(pmax));
          }
          const bool grow = m_tile > m_run[rb] + RESCALE_GAP;
          const float m_new = grow ? m_tile : m_run[rb];
          const float alpha = fast_exp2(m_run[rb] - m_new);
          m_run[rb] = m_new;
          thr[rb] = (m_new + RESCALE_GAP) / a.c;
          l_s[rb] *= alpha;
          l_c[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[rb][db] *= alpha;
          if (lost) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int e = 0; e < 4; ++e) s[rb][kb][e] = fast_exp2(fmaf(s[rb][kb][e], a.c, -m_new));
          } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[rb][kb] *= alpha;
          }
          ls = row_part(rb);
        }
        lsum[rb] = ls;
      } else {
        if constexpr (masked) {
          // key j0 + 8 grp + off is past this row when off > lim
          const int lim = row_pos[rb] - j0 - 8 * grp;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (32 * (kb >> 1) + 4 * (kb & 1) + e > lim) s[rb][kb][e] = -INFINITY;
        }
        const float m0 = max3f(s[rb][0][0], s[rb][0][1], s[rb][0][2]);
        const float m1 = max3f(s[rb][0][3], s[rb][1][0], s[rb][1][1]);
        const float m2 = max3f(s[rb][1][2], s[rb][1][3], s[rb][2][0]);
        const float m3 = max3f(s[rb][2][1], s[rb][2][2], s[rb][2][3]);
        const float m4 = max3f(s[rb][3][0], s[rb][3][1], s[rb][3][2]);
        // this lane's 16 logits of the row: a row grows exactly when one of
        // its four lanes does, so the cross-lane maximum is only formed on
        // the (rare) tiles where some lane of the wave grows
        const float lmax = max2f(max3f(m0, m1, m2), max3f(m3, m4, s[rb][3][3]));
        if (__builtin_amdgcn_ballot_w64(lmax > thr[rb])) {
          const float m_tile = row_group_max(lmax) * a.c;
          const bool grow = m_tile > m_run[rb] + RESCALE_GAP;
          const float m_new = grow ? m_tile : m_run[rb];
          const float alpha = fast_exp2(m_run[rb] - m_new);
          m_run[rb] = m_new;
          thr[rb] = (m_new + RESCALE_GAP) / a.c;
          l_s[rb] *= alpha;
          l_c[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[rb][db] *= alpha;
        }
        const float neg_m = -m_run[rb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[rb][kb][e] = fast_exp2(fmaf(s[rb][kb][e], a.c, neg_m));
        lsum[rb] = row_part(rb);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pu[rb][st][e] = (__bf16)s[rb][2 * st][e];
          pu[rb][st][4 + e] = (__bf16)s[rb][2 * st + 1][e];
        }
    }
  };

  // one tile step; stage_c = t % 2 (known at compile time in the unrolled
  // loop over open tiles, at run time on the few diagonal tiles): K(t) and
  // Vt(t) live in stage t % 2, Vt(t - 1) in the other one
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using SR = std::integral_constant<int, -1>;
  // a wave's share of the loads issued right after barrier t
  auto loads = [&](int t, int st) __attribute__((always_inline)) {
    if (t + 1 < n_tiles) issue_k(t + 1, st ^ 1);
    issue_v(t, st);
  };
  auto step = [&](int t, auto stage_c, auto masked_c, auto first_c) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
    const int ST = SC >= 0 ? SC : (t & 1);
    if (lead) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();                                  // barrier t
      loads(t, ST);
    } else if (decltype(first_c)::value) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();                                  // barrier 0
      loads(0, 0);
    }
    if constexpr (!decltype(first_c)::value) {
      if constexpr (SC >= 0) pv(std::integral_constant<int, SC ^ 1>{});   // tile t - 1
      else if (ST) pv(S0{});
      else pv(S1{});
    }
    if constexpr (SC >= 0) qk(stage_c);
    else if (ST) qk(S1{});
    else qk(S0{});
    if (!lead) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();                                  // barrier t + 1
      if (t + 1 < n_tiles) loads(t + 1, ST ^ 1);
    }
    softmax(t, masked_c, std::integral_constant<bool, !decltype(masked_c)::value &&
                                                     !decltype(first_c)::value>{});
  };
  using Open = std::false_type;
  using Diag = std::true_type;
  using First = std::true_type;
  using Later = std::false_type;
  // tiles below n_full have no key past any row here: no causal mask
  if (n_tiles > 0) {
    issue_k(0, 0);
    if (n_full > 0) step(0, S0{}, Open{}, First{});
    else step(0, S0{}, Diag{}, First{});
  }
  int t = 1;
  if (t < n_full && (t & 1)) step(t++, S1{}, Open{}, Later{});
  for (; t + 1 < n_full; t += 2) {
    step(t, S0{}, Open{}, Later{});
    step(t + 1, S1{}, Open{}, Later{});
  }
  if (t < n_full) step(t++, S0{}, Open{}, Later{});
  for (; t < n_tiles; ++t) step(t, SR{}, Diag{}, Later{});
  // the last tile's PV product, after barrier n_tiles (the leading group's
  // here, the other group's in its last step)
  if (n_tiles > 0) {
    if (lead) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    }
    if ((n_tiles - 1) & 1) pv(S1{});
    else pv(S0{});
  }

#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    float l = l_s[rb] - l_c[rb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = r0 + wave * 16 * RBW + rb * 16 + l16;
    if (r >= R) continue;
    const int i = r / G, hh = r - (r / G) * G;
    const int h = g * G + hh;
    const float inv = 1.f / l;
    __bf16* orow = oseq + ((size_t)i * a.h_q + h) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      __attribute__((ext_vector_type(4))) __bf16 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(acc[rb][db][e] * inv);
      *reinterpret_cast<decltype(w4)*>(orow + db * 16) = w4;
    }
    if (grp == 0) {
      const size_t si = (size_t)h * nq + i;
      stats[si] = m_run[rb];
      stats[plane + si] = l;
      stats[2 * plane + si] = 1.f / l;
      if (lse) lse[si] = (m_run[rb] + log2f(l)) * LN2;
    }
  }
}

bool prefill_uses_vt(const Shape& s) { return s.bf16 && s.head_dim == D; }

int prefill_rows_per_tile() { return 16 * 2 * FWD_WAVES; }


int vt_keys_for(int n_kv) { return (n_kv + TK - 1) / TK * TK; }

hipError_t launch_attn_fwd_prefill_generic(const FwdPlan& p, hipStream_t st);

hipError_t launch_v_transpose(const FwdPlan& p, hipStream_t st) {
  if (!prefill_uses_vt(p.s) || !p.vt) return hipSuccess;
  const int vt_tiles = p.vt_keys / TK;
  const unsigned tgrid = (unsigned)((size_t)p.s.batch * p.s.h_kv * vt_tiles);
  hipLaunchKernelGGL(transpose_v_kernel, dim3(tgrid), dim3(256), 0, st,
                     reinterpret_cast<const __bf16*>(p.v), reinterpret_cast<__bf16*>(p.vt),
                     p.s.n_kv, p.s.h_kv, vt_tiles);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_prefill(const FwdPlan& p, hipStream_t st) {
  if (!prefill_uses_vt(p.s) || !p.vt) return launch_attn_fwd_prefill_generic(p, st);
  const int vt_tiles = p.vt_keys / TK;
  Fwd2Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.vt = reinterpret_cast<const __bf16*>(p.vt);
  a.o = reinterpret_cast<__bf16*>(p.o);
  a.stats = p.stats; a.lse = p.lse;
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.vt_tiles = vt_tiles; a.c = p.s.scale_log2;
  const int G = a.h_q / a.h_kv;
  // two 16-row blocks per wave at two waves per SIMD measured best on the
  // 1M-context workload: 48 rows fit the registers only with the softmax
  // split into 32-key halves, which ran slower; 64 rows at one wave per
  // SIMD lose more to latency than they save in LDS traffic; eight waves
  // sharing each tile beat four waves by about 3 %
  constexpr int RBW = 2, NWV = FWD_WAVES;
  constexpr int rows = 16 * RBW * NWV;
  static_assert(2 * STAGE_BYTES <= 65536, "the two-stage ring is a static LDS array");
  a.n_rt = (a.n_q * G + rows - 1) / rows;
  dim3 grid((unsigned)((size_t)a.n_rt * a.B * a.h_kv));
  if (p.vl) {
    a.vl = *p.vl;
    grid = dim3((unsigned)((size_t)a.vl.tile0[a.vl.n] * a.h_kv));
    if (a.vl.tile0[a.vl.n] == 0) return hipSuccess;
  }
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<RBW, NWV>), grid, dim3(64 * NWV), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
