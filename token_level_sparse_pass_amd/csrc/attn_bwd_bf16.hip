// dQ of the full layer's backward pass, specialised for bf16 and head dim
// 128 (fine-tuning at long context; HySparse2 pages: "Xiaomi Unveils
// HySparse2 for Faster Long-Context AI", section "Performance Gains: Cost,
// Speed, and Long-Context Capabilities"). Same contract as the dQ kernel of
// attn_bwd.hip:
//   P = 2^(t * c - lse2),  dP = dO V^T,  dS = P * (dP - Delta),  dQ = scale dS K
// with t the raw logit q.k, c = scale * log2(e) and lse2 = lse * log2(e).
//
// Laid out like the forward pass-1 kernel: a work-group owns 256 rows
// (query, head-of-group pairs) of one (sequence, KV head), eight waves of
// two 16-row MFMA blocks, two waves per SIMD; each 64-key tile of K, V and
// of a transposed copy of K (Kt[b][g][tile][d][64 keys], written once per
// call by the V-layout kernel) goes straight into LDS through a two-stage
// ring, XOR-swizzled so the fragment reads are conflict-free. Per key block:
//   S^T  = K . Q^T,  dP^T = V . dO^T    A = K / V rows (LDS), B = Q / dO (regs)
//   dS^T = P^T * (dP^T - Delta)          in the accumulators, packed to bf16
// and per 32-key step dQ^T += Kt . dS^T (A = Kt rows (LDS), B = dS^T), with
// the keys of a tile in the permuted order that gives each lane's B operand
// 8 consecutive keys. Tiles below the diagonal run a copy of the body
// without the causal mask.
#include "hs2_device.h"
#include "hs2_launch.h"

#include <type_traits>

namespace hs2 {

namespace {

constexpr int TK = 64;                        // keys per tile
constexpr int D = 128;
constexpr int KT_BYTES = TK * D * 2;          // 16 KB per tensor tile
constexpr int V_OFF = KT_BYTES;               // stage layout: K, V, Kt
constexpr int KT_OFF = 2 * KT_BYTES;
constexpr int STAGE_BYTES = 3 * KT_BYTES;
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

// chunk swizzles: K and V tile rows are 256 B (16 chunks), Kt rows 128 B (8)
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
__device__ __forceinline__ int tswz(int row) { return (row >> 1) & 7; }

// key held in MFMA row m of key block kb (lane group q of the B operand of
// the dQ product then owns keys 32 * (kb / 2) + 8q .. +7 of the tile)
__device__ __forceinline__ int tile_key(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct DqArgs {
  const __bf16* q; const __bf16* k; const __bf16* v; const __bf16* kt; const __bf16* dout;
  const float* lse; const float* delta;
  __bf16* dq;
  int B, n_q, n_kv, h_q, h_kv, n_rt, kt_tiles;
  float scale, c;
};

}  // namespace

template <int RBW, int NWV>
__global__ __launch_bounds__(64 * NWV, 2) void attn_bwd_dq_bf16_kernel(DqArgs a) {
  using OP = Op<__bf16, D>;
  constexpr int ROWS = 16 * RBW * NWV;                  // rows per work-group
  constexpr int CPT = 1024 / (64 * NWV);                // 16-byte chunks per thread per tensor
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.h_q / a.h_kv;
  const uint32_t lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int rt = a.n_rt - 1 - (int)(lid % a.n_rt);      // heavy tiles first
  const int bg = lid / a.n_rt;
  const int b = bg % a.B;
  const int g = bg / a.B;

  const int R = a.n_q * G;
  const int q_off = a.n_kv - a.n_q;
  const int r0 = rt * ROWS;
  const int i_hi = min(a.n_q - 1, (r0 + ROWS - 1) / G);
  const int p_lo = q_off + r0 / G;
  const int p_hi = q_off + i_hi;
  const int n_tiles = (p_hi + TK) / TK;
  const int n_full = (p_lo + 1) / TK;                   // tiles with no masked key

  const size_t kstride = (size_t)a.h_kv * D;
  const __bf16* kseq = a.k + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const __bf16* vseq = a.v + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const __bf16* ktseq = a.kt + ((size_t)b * a.h_kv + g) * a.kt_tiles * (size_t)(D * TK);

  // ---- the rows' Q and dO fragments and statistics ----
  Frag<__bf16, D> qf[RBW], df[RBW];
  float l2[RBW], dl[RBW];
  int row_pos[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * 16 * RBW + rb * 16 + l16;
    if (r < R) {
      const int i = r / G, h = g * G + (r - (r / G) * G);
      const size_t off = (((size_t)b * a.n_q + i) * a.h_q + h) * D;
      load_slice<__bf16, D>(qf[rb], a.q + off, lane);
      load_slice<__bf16, D>(df[rb], a.dout + off, lane);
      const size_t si = ((size_t)b * a.h_q + h) * a.n_q + i;
      l2[rb] = a.lse[si] * LOG2E;
      dl[rb] = a.delta[si];
      row_pos[rb] = q_off + i;
    } else {
      zero_slice<__bf16, D>(qf[rb]);
      zero_slice<__bf16, D>(df[rb]);
      l2[rb] = INFINITY;                                // P = 0
      dl[rb] = 0.f;
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
      const size_t row = (size_t)min(j0 + r, a.n_kv - 1) * kstride + c * 8;
      const __bf16* ks = kseq + row;
      const __bf16* vs = vseq + row;
      __builtin_amdgcn_global_load_lds(ks, (lds_void*)(base + (wave * CPT + t) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vs, (lds_void*)(base + V_OFF + (wave * CPT + t) * 1024), 16,
                                       0, 0);
    }
    const __bf16* ktile = ktseq + (size_t)tile * (D * TK);
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
      const int slot = (wave * CPT + t) * 64 + lane;
      const int d = slot >> 3, pc = slot & 7;
      const int c = pc ^ tswz(d);
      const __bf16* ts = ktile + d * TK + c * 8;
      __builtin_amdgcn_global_load_lds(ts, (lds_void*)(base + KT_OFF + (wave * CPT + t) * 1024), 16,
                                       0, 0);
    }
  };

  f32x4 acc[RBW][8];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets: key blocks 0, 1 (blocks 2, 3 hold rows 32 further,
  // same swizzle, 8 KB on); Kt rows 16 db + l16 of each 32-key step (row
  // 16 db + l16 is db * 2 KB on)
  int koff[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = tile_key(kb, l16);
#pragma unroll
    for (int u = 0; u < 4; ++u) koff[kb][u] = row * 256 + (((4 * grp + u) ^ kswz(row)) << 4);
  }
  int toff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) toff[st] = KT_OFF + l16 * 128 + (((4 * st + grp) ^ tswz(l16)) << 4);

  if (n_tiles > 0) issue(0, 0);
  auto step = [&](int t, auto stage_c, auto masked_c) {
    constexpr int STAGE_C = decltype(stage_c)::value;       // -1: runtime
    constexpr bool masked = decltype(masked_c)::value;
    const int stage = STAGE_C >= 0 ? STAGE_C : (t & 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // the other stage held tile t - 1, which every wave finished reading
    // before the barrier above
    if (t + 1 < n_tiles) issue(t + 1, stage ^ 1);
    const char* base = smem + stage * STAGE_BYTES;
    const int j0 = t * TK;

    // dS^T of the four key blocks, packed for the dQ product: lane group
    // grp of step st holds keys 32 st + 8 grp .. +7
    bf16x8 pu[RBW][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 kf[4], vf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int o = koff[kb & 1][u] + (kb >> 1) * 8192;
        kf[u] = *reinterpret_cast<const bf16x8*>(base + o);
        vf[u] = *reinterpret_cast<const bf16x8*>(base + V_OFF + o);
      }
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) s = OP::mma(kf[u], qf[rb].u[u], s);
#pragma unroll
        for (int u = 0; u < 4; ++u) dp = OP::mma(vf[u], df[rb].u[u], dp);
        int lim = 0;
        if constexpr (masked) lim = row_pos[rb] - j0 - 8 * grp;   // key j0 + 8 grp + off > row
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = fast_exp2(fmaf(s[e], a.c, -l2[rb]));
          if constexpr (masked) {
            if (32 * (kb >> 1) + 4 * (kb & 1) + e > lim) p = 0.f;
          }
          pu[rb][kb >> 1][(kb & 1) * 4 + e] = (__bf16)(p * (dp[e] - dl[rb]));
        }
      }
    }

    // dQ^T += Kt . dS^T; the Kt fragments (position 8 st + db) stream two
    // positions ahead of their MFMAs
    auto tfrag = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(base + toff[i >> 3] + (i & 7) * 2048);
    };
    bf16x8 tf[3];
    tf[0] = tfrag(0);
    tf[1] = tfrag(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) tf[(i + 2) % 3] = tfrag(i + 2);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        acc[rb][i & 7] = OP::mma(tf[i % 3], pu[rb][i >> 3], acc[rb][i & 7]);
    }
  };
  // tiles below n_full need no causal mask; the loop is unrolled by two so
  // each stage's LDS offsets are immediates of the read instructions
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    step(t, S0{}, std::false_type{});
    step(t + 1, S1{}, std::false_type{});
  }
  if (t < n_full) step(t++, S0{}, std::false_type{});
  for (; t < n_tiles; ++t) step(t, std::integral_constant<int, -1>{}, std::true_type{});

  // lane holds dQ^T[d = 16 db + 4 grp + e][row l16]
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * 16 * RBW + rb * 16 + l16;
    if (r >= R) continue;
    const int i = r / G, h = g * G + (r - (r / G) * G);
    __bf16* orow = a.dq + (((size_t)b * a.n_q + i) * a.h_q + h) * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      __attribute__((ext_vector_type(4))) __bf16 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(acc[rb][db][e] * a.scale);
      *reinterpret_cast<decltype(w4)*>(orow + db * 16) = w4;
    }
  }
}

bool bwd_dq_uses_bf16_kernel(const Shape& s) { return s.bf16 && s.head_dim == D; }

hipError_t launch_bwd_dq_bf16(const BwdPlan& p, hipStream_t st) {
  constexpr int RBW = 2, NWV = 8;
  constexpr int rows = 16 * RBW * NWV;
  constexpr int smem_bytes = 2 * STAGE_BYTES;
  DqArgs a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.kt = reinterpret_cast<const __bf16*>(p.kt);
  a.dout = reinterpret_cast<const __bf16*>(p.dout);
  a.lse = p.lse; a.delta = p.delta;
  a.dq = reinterpret_cast<__bf16*>(p.dq);
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.kt_tiles = vt_keys_for(p.s.n_kv) / TK;
  a.scale = p.scale; a.c = p.s.scale_log2;
  const int G = a.h_q / a.h_kv;
  a.n_rt = (a.n_q * G + rows - 1) / rows;
  struct DqLdsTag {};
  {
    const hipError_t e = ensure_dynamic_lds<DqLdsTag>(
        (const void*)attn_bwd_dq_bf16_kernel<RBW, NWV>, smem_bytes);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((size_t)a.n_rt * a.B * a.h_kv));
  hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<RBW, NWV>), grid, dim3(64 * NWV), smem_bytes, st, a);
  return hipGetLastError();
}

}  // namespace hs2
