// Pass 1 of the full layer, specialised for bf16 and head dim 128 (the
// long-context workloads). Same contract as attn_fwd.hip: causal GQA
// attention over the shared K/V plus per-(query, head) statistics
// (m2, l) and LSE.
//
// Differences from the generic kernel, all aimed at keeping the SIMD's
// issue slots on MFMAs (with two waves per SIMD issuing both, every VALU
// instruction in the loop costs MFMA time: about 2-3 cycles each, measured
// with MFMA and FMA streams interleaved in each wave):
//  * V is transposed once per call into a tile-major copy in the workspace,
//    Vt[b][g][tile][d][64 keys], so the PV product reads its operands with
//    16-byte LDS loads instead of transposing in registers;
//  * K and Vt tiles go straight from global memory into LDS
//    (global_load_lds_dwordx4) through a two-stage ring (the next tile
//    loads while this one is used), with XOR-swizzled 16-byte chunks so
//    the MFMA operand reads are free of bank conflicts; the tile loop is
//    unrolled by two so each stage's LDS offsets are immediates of the
//    read instructions, and tiles that need no causal mask run a copy of
//    the loop body without one;
//  * row maxima use three-input max instructions and the gfx950 permlane
//    swaps (no LDS round trip for the cross-row step); this file is built
//    with -fno-honor-nans so that fmaxf does not first quiet every operand
//    (the kernel never sees a NaN: masked logits are -inf);
//  * the keys of a 64-key tile are assigned to MFMA rows in a permuted order
//    such that the P^T operand of each lane covers 8 consecutive keys;
//  * the running max is only moved (and O rescaled) when it grows by more
//    than 2^8, so the rescale multiply almost never runs; exponents are
//    formed with one FMA (logit * c - m) from the raw MFMA result;
//  * the causal mask is applied only on tiles that reach the diagonal.
// Rows, as in the generic kernel, are (query, head-of-group) pairs: RBW
// 16-row MFMA blocks per wave, eight waves (two per SIMD) per work-group,
// all sharing each tile in LDS. Each wave reads a whole K and V^T tile from
// LDS per 64 keys (512 B per MFMA); the counters put the LDS pipe at under
// half of its cycles, so the loop is bound by instruction issue, not LDS.
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
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void;

// chunk swizzles: K tile rows are 256 B (16 chunks), Vt rows 128 B (8 chunks)
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
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
  constexpr int CPT = 1024 / (64 * NWV);                // 16-byte chunks per thread per tensor
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  // ---- tile loads straight into LDS ----
  auto issue = [&](int tile, int stage) {
    char* base = smem + stage * STAGE_BYTES;
    const int j0 = tile * TK;
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
      const int slot = (wave * CPT + t) * 64 + lane;
      const int r = slot >> 4, pc = slot & 15;
      const int c = pc ^ kswz(r);
      const int key = min(j0 + r, nkv - 1);
      const __bf16* src = kseq + (size_t)key * kstride + c * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + (wave * CPT + t) * 1024), 16, 0, 0);
    }
    const __bf16* vsrc = vtseq + (size_t)tile * (D * TK);
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
      const int slot = (wave * CPT + t) * 64 + lane;
      const int d = slot >> 3, pc = slot & 7;
      const int c = pc ^ vswz(d);
      __builtin_amdgcn_global_load_lds(
          vsrc + d * TK + c * 8, (lds_void*)(base + KT_BYTES + (wave * CPT + t) * 1024), 16, 0, 0);
    }
  };

  float m_run[RBW];
  float l_s[RBW], l_c[RBW];                             // compensated row sums
  f32x4 acc[RBW][8];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m_run[rb] = -1e30f;
    l_s[rb] = 0.f;
    l_c[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS offsets that do not change between tiles
  int koff[4][4];                                       // [kb][unit] byte offset in K tile
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int row = tile_key(kb, l16);
#pragma unroll
    for (int u = 0; u < 4; ++u) koff[kb][u] = row * 256 + (((4 * grp + u) ^ kswz(row)) << 4);
  }
  int voff[2][8];                                       // [step][db] byte offset in Vt tile
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = db * 16 + l16;
      voff[st][db] = KT_BYTES + d * 128 + (((4 * st + grp) ^ vswz(d)) << 4);
    }

  // two-stage ring: tile t + 1 is loaded into the other stage while tile t
  // is used; the loop is unrolled by two so each stage's LDS offsets are
  // compile-time constants folded into the LDS read instructions
  if (n_tiles > 0) issue(0, 0);
  auto step = [&](int t, auto stage_c, auto masked_c) {
    constexpr int STAGE_C = decltype(stage_c)::value;       // -1: runtime
    constexpr bool masked = decltype(masked_c)::value;
    const int STAGE = STAGE_C >= 0 ? STAGE_C : (t & 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // the other stage held tile t - 1, which every wave finished reading
    // before the barrier above
    if (t + 1 < n_tiles) issue(t + 1, STAGE ^ 1);
    const char* base = smem + STAGE * STAGE_BYTES;
    const int j0 = t * TK;

    // logits^T for 4 key blocks x 2 row blocks; the K fragments of block
    // kb + 1 are read from LDS while block kb's MFMAs run
    f32x4 s[RBW][4];
    bf16x8 kf[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kf[0][u] = *reinterpret_cast<const bf16x8*>(base + koff[0][u]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kf[cur ^ 1][u] = *reinterpret_cast<const bf16x8*>(base + koff[kb + 1][u]);
      }
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) x = OP::mma(kf[cur][u], qf[rb].u[u], x);
        s[rb][kb] = x;
      }
    }
    // V fragments of the first PV step, read during the softmax arithmetic
    bf16x8 vf0[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) vf0[db] = *reinterpret_cast<const bf16x8*>(base + voff[0][db]);

    bf16x8 pu[RBW][2];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
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
      const float tmax = row_group_max(max2f(max3f(m0, m1, m2), max3f(m3, m4, s[rb][3][3])));
      const float m_tile = tmax * a.c;
      const bool grow = m_tile > m_run[rb] + RESCALE_GAP;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_tile : m_run[rb];
        const float alpha = fast_exp2(m_run[rb] - m_new);
        m_run[rb] = m_new;
        l_s[rb] *= alpha;
        l_c[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[rb][db] *= alpha;
      }
      const float neg_m = -m_run[rb];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(fmaf(s[rb][kb][e], a.c, neg_m));
          s[rb][kb][e] = pe;
          psum += pe;
        }
      // compensated add of this tile's row sum
      const float y = psum - l_c[rb];
      const float tt = l_s[rb] + y;
      l_c[rb] = (tt - l_s[rb]) - y;
      l_s[rb] = tt;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pu[rb][st][e] = (__bf16)s[rb][2 * st][e];
          pu[rb][st][4 + e] = (__bf16)s[rb][2 * st + 1][e];
        }
    }

    // O^T += V^T . P^T (step 1's V fragments are read during step 0)
    bf16x8 vf1[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      vf1[db] = *reinterpret_cast<const bf16x8*>(base + voff[1][db]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) acc[rb][db] = OP::mma(vf0[db], pu[rb][0], acc[rb][db]);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) acc[rb][db] = OP::mma(vf1[db], pu[rb][1], acc[rb][db]);
  };
  // tiles below n_full have no key past any row here: no causal mask
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Open = std::false_type;
  using Diag = std::true_type;
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    step(t, S0{}, Open{});
    step(t + 1, S1{}, Open{});
  }
  if (t < n_full) step(t++, S0{}, Open{});
  for (; t < n_tiles; ++t) step(t, std::integral_constant<int, -1>{}, Diag{});

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
  constexpr int smem_bytes = 2 * STAGE_BYTES;
  struct FwdLdsTag {};
  if (smem_bytes > 65536) {
    const hipError_t e = ensure_dynamic_lds<FwdLdsTag>(
        (const void*)attn_fwd_bf16_kernel<RBW, NWV>, smem_bytes);
    if (e != hipSuccess) return e;
  }
  a.n_rt = (a.n_q * G + rows - 1) / rows;
  dim3 grid((unsigned)((size_t)a.n_rt * a.B * a.h_kv));
  if (p.vl) {
    a.vl = *p.vl;
    grid = dim3((unsigned)((size_t)a.vl.tile0[a.vl.n] * a.h_kv));
    if (a.vl.tile0[a.vl.n] == 0) return hipSuccess;
  }
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<RBW, NWV>), grid, dim3(64 * NWV), smem_bytes, st,
                     a);
  return hipGetLastError();
}

}  // namespace hs2
