// dQ and dK/dV of the full layer's backward pass, specialised for bf16 and
// head dim 128 (fine-tuning at long context; HySparse2 pages: "Xiaomi
// Unveils HySparse2 for Faster Long-Context AI", section "Performance
// Gains: Cost, Speed, and Long-Context Capabilities"). Same contract as the
// kernels of attn_bwd.hip:
//   P = 2^(t * c - lse2),  dP = dO V^T,  dS = P * (dP - Delta),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// with t the raw logit q.k, c = scale * log2(e) and lse2 = lse * log2(e).
// The dK/dV kernel and its row-layout kernel follow the dQ kernel below.
//
// The dQ kernel is laid out like the forward pass-1 kernel: a work-group owns 256 rows
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

// chunk swizzles: K and V tile rows are 256 B (16 chunks), Kt rows 128 B (8).
// A 16-byte read of 64 lanes is served 32 lanes at a time from 128 banks
// (512 B), so rows of equal parity share banks. kswz (rows tile_key(kb, l16),
// built from row bits 0, 1, 3, 4 with bits 0 and 3 in swapped places) and
// rswz (rows 16 rb + l16: the low four bits with bits 0 and 2 swapped) put
// the 32 chunks a half wave reads on distinct bank groups.
__device__ __forceinline__ int kswz(int row) {
  return ((row >> 3) & 1) | (row & 2) | ((row & 1) << 2) | (((row >> 4) & 1) << 3);
}
__device__ __forceinline__ int rswz(int row) { return (row & 10) | ((row & 1) << 2) | ((row >> 2) & 1); }
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
  // longest first over the whole grid (row tile descending, every
  // (sequence, KV head) at each step), as in the forward kernel
  const int rt = a.n_rt - 1 - (int)(blockIdx.x / (a.B * a.h_kv));
  const int bg = blockIdx.x % (a.B * a.h_kv);
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

// ---------------------------------------------------------------------------
// dK, dV of the full layer (bf16, head dim 128). A work-group owns 128 keys
// of one (sequence, KV head) and walks the rows (query, head-of-group pairs)
// that see them in 64-row tiles, from the last tile down. Per tile four
// tensors come straight into a two-stage LDS ring: the Q and dO rows (for
// S = Q K^T and dP = dO V^T, A = rows, B = keys) and their transposed
// copies Qt, dOt [d][64 rows] written once per call by
// bwd_rows_layout_kernel, so that the row contractions
//   dV^T += dO^T P,   dK^T += Q^T dS          (A = Qt / dOt, B = P / dS)
// read one 16-byte fragment per MFMA with no register transposes. Within
// each 32-row half of a tile the transposed copies hold row
// 16 (x / 4) + 4 q + x % 4 at position 8 q + x: the rows a lane of group q
// holds in its S accumulators, in slot order.
// ---------------------------------------------------------------------------

namespace {

constexpr int TR = 64;                               // rows per tile
constexpr int ROWS_T_BYTES = TR * D * 2;             // 16 KB per tensor tile
constexpr int DK_QR = 0, DK_DR = ROWS_T_BYTES, DK_QT = 2 * ROWS_T_BYTES, DK_DT = 3 * ROWS_T_BYTES;
constexpr int DK_STAGE = 4 * ROWS_T_BYTES;           // stats of both stages follow the ring
constexpr int DK_STATS = 2 * DK_STAGE;
constexpr int DK_SMEM = DK_STATS + 2 * 2 * TR * 4;

// tile row (in 0 .. 63) stored at position pos of a transposed tile
__device__ __forceinline__ int trow_of_pos(int pos) {
  const int x = pos & 7, q = (pos >> 3) & 3;
  return (pos & 32) + 16 * (x >> 2) + 4 * q + (x & 3);
}

struct RowsArgs {
  const __bf16* q; const __bf16* dout;
  const float* lse; const float* delta;
  __bf16* qt; __bf16* dot; float* rst;
  int n_q, h_q, h_kv, n_rt;
};

struct DkdvArgs {
  const __bf16* q; const __bf16* dout; const __bf16* k; const __bf16* v;
  const __bf16* qt; const __bf16* dot; const float* rst;
  const void* acc_k; const void* acc_v;
  bool acc_fixed; const float* acc_scale;
  __bf16* dk; __bf16* dv;
  int B, n_q, n_kv, h_q, h_kv, n_rt, n_kt;
  int q64, r64;                                       // 64 = q64 * G + r64
  float scale, c;
};

}  // namespace

// Q and dO of one (sequence, KV head, 64-row tile) transposed to [d][64]
// (position order above, zero past the last row), and the tile's
// lse * log2(e) (+inf past the last row) and Delta, as rst[tile][2][64].
__global__ __launch_bounds__(256) void bwd_rows_layout_kernel(RowsArgs a) {
  __shared__ uint16_t tile[TR][D + 8];
  const int G = a.h_q / a.h_kv;
  const int R = a.n_q * G;
  const int t = blockIdx.x % a.n_rt;
  const int bg = blockIdx.x / a.n_rt;
  const int g = bg % a.h_kv;
  const int b = bg / a.h_kv;
  const size_t tile_id = (size_t)bg * a.n_rt + t;
#pragma unroll 1
  for (int which = 0; which < 2; ++which) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(which ? a.dout : a.q);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = threadIdx.x + 256 * it;
      const int rr = u >> 4, c = u & 15;
      const int r = t * TR + rr;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r < R) {
        const int i = r / G, h = r - (r / G) * G;
        val = *reinterpret_cast<const uint4*>(src + (((size_t)b * a.n_q + i) * a.h_q + g * G + h) * D +
                                              c * 8);
      }
      *reinterpret_cast<uint4*>(&tile[rr][c * 8]) = val;
    }
    __syncthreads();
    uint16_t* dst = reinterpret_cast<uint16_t*>(which ? a.dot : a.qt) + tile_id * (D * TR);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = threadIdx.x + 256 * it;          // 1024 chunks of 8 positions
      const int d = u >> 3, c = u & 7;
      uint16_t e[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) e[x] = tile[trow_of_pos(8 * c + x)][d];
      uint4 w;
      w.x = e[0] | ((uint32_t)e[1] << 16);
      w.y = e[2] | ((uint32_t)e[3] << 16);
      w.z = e[4] | ((uint32_t)e[5] << 16);
      w.w = e[6] | ((uint32_t)e[7] << 16);
      *reinterpret_cast<uint4*>(dst + d * TR + c * 8) = w;
    }
    __syncthreads();
  }
  if (threadIdx.x < TR) {
    const int r = t * TR + threadIdx.x;
    float l2 = INFINITY, dl = 0.f;                    // P = 0 past the last row
    if (r < R) {
      const int i = r / G, h = r - (r / G) * G;
      const size_t si = ((size_t)b * a.h_q + g * G + h) * a.n_q + i;
      l2 = a.lse[si] * LOG2E;
      dl = a.delta[si];
    }
    a.rst[tile_id * (2 * TR) + threadIdx.x] = l2;
    a.rst[tile_id * (2 * TR) + TR + threadIdx.x] = dl;
  }
}

// dK, dV with paired waves: waves 0..3 hold the K rows of 32 keys each and
// accumulate dV^T, waves 4..7 hold the V rows of the same keys and
// accumulate dK^T, so each wave keeps 32 keys' operands and one set of
// accumulators (96 registers) where one wave holding both would need 192.
// Per 64-row tile, a K wave forms S = Q K^T and P, hands P (bf16, in its
// accumulator lane order) to its V wave through LDS and adds dO^T P; the V
// wave forms dP = dO V^T, then dS = P (dP - Delta) and adds Q^T dS. Each
// LDS fragment read then feeds two key blocks' MFMAs.
constexpr int DKP_X = DK_SMEM;                        // P hand-over: [pair][st][kb][lane] x 16 B
constexpr int DKP_SMEM = DKP_X + 4 * 2 * 2 * 64 * 16;
constexpr int DKP_KEYS = 128;                         // keys per work-group

__global__ __launch_bounds__(512, 2) void attn_bwd_dkdv_bf16_pair_kernel(DkdvArgs a) {
  using OP = Op<__bf16, D>;
  constexpr int NWV = 8, KB = 2;
  constexpr int KT = 16 * KB * (NWV / 2);
  static_assert(KT == DKP_KEYS, "keys per work-group");
  constexpr int CPT = 1024 / (64 * NWV);
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int l16 = lane & 15;
  const bool vwave = wave >= 4;                       // V rows, dK; else K rows, dV
  const int pair = wave & 3;
  const int G = a.h_q / a.h_kv;
  const int q_off = a.n_kv - a.n_q;
  // longest first over the whole grid: key tile 0 (seen by the most rows)
  // of every (sequence, KV head), then tile 1, ...
  const int kt = (int)(blockIdx.x / (a.B * a.h_kv));
  const int bg = (int)(blockIdx.x % (a.B * a.h_kv));
  const int b = bg % a.B;
  const int g = bg / a.B;
  const int j0 = kt * KT;
  const int jw = j0 + pair * KB * 16;

  // ---- the pair's keys: K (or V) rows as B operands, one accumulator set ----
  const size_t kstride = (size_t)a.h_kv * D;
  Frag<__bf16, D> kv[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = jw + kb * 16 + l16;
    if (j < a.n_kv) {
      const size_t off = ((size_t)b * a.n_kv + j) * kstride + (size_t)g * D;
      load_slice<__bf16, D>(kv[kb], (vwave ? a.v : a.k) + off, lane);
    } else {
      zero_slice<__bf16, D>(kv[kb]);
    }
  }
  f32x4 acc[KB][8];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- row tiles: rows that see key j0 onwards, the last tile first ----
  const int rt_begin = (max(0, j0 - q_off) * G) / TR;
  const int i_need = j0 + KT - 1 - q_off;             // a tile is unmasked when its
  int t_u = i_need <= 0 ? 0 : (int)(((int64_t)i_need * G + TR - 1) / TR);   // first row sees all keys
  t_u = min(max(t_u, rt_begin), a.n_rt);
  const int n_tiles = a.n_rt - rt_begin;
  const int n_unm = a.n_rt - t_u;

  // per-slot (query, head) of the row chunks this thread loads, for the
  // tile issued next; stepped down by 64 rows per tile
  const size_t tile0 = (size_t)(b * a.h_kv + g) * a.n_rt;
  int si_[CPT], sh_[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int slot = (wave * CPT + c) * 64 + lane;
    const int r = (a.n_rt - 1) * TR + (slot >> 4);
    si_[c] = r / G;
    sh_[c] = r - si_[c] * G;
  }
  const __bf16* qseq = a.q + ((size_t)b * a.n_q * a.h_q + (size_t)g * G) * D;
  const __bf16* dseq = a.dout + ((size_t)b * a.n_q * a.h_q + (size_t)g * G) * D;

  auto issue = [&](int tile, int stage) {
    char* base = smem + stage * DK_STAGE;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int slot = (wave * CPT + c) * 64 + lane;
      const int rr = slot >> 4, pc = slot & 15;
      const int ch = pc ^ rswz(rr);
      const size_t row = ((size_t)min(si_[c], a.n_q - 1) * a.h_q + sh_[c]) * D + ch * 8;
      const __bf16* qs = qseq + row;
      const __bf16* ds = dseq + row;
      __builtin_amdgcn_global_load_lds(qs, (lds_void*)(base + DK_QR + (wave * CPT + c) * 1024), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds(ds, (lds_void*)(base + DK_DR + (wave * CPT + c) * 1024), 16, 0,
                                       0);
      // the same slot, 64 rows lower, for the next tile
      sh_[c] -= a.r64;
      si_[c] -= a.q64;
      if (sh_[c] < 0) { sh_[c] += G; si_[c] -= 1; }
    }
    const size_t toff_g = (tile0 + tile) * (size_t)(D * TR);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int slot = (wave * CPT + c) * 64 + lane;
      const int d = slot >> 3, pc = slot & 7;
      const int ch = pc ^ tswz(d);
      const __bf16* qs = a.qt + toff_g + d * TR + ch * 8;
      const __bf16* ds = a.dot + toff_g + d * TR + ch * 8;
      __builtin_amdgcn_global_load_lds(qs, (lds_void*)(base + DK_QT + (wave * CPT + c) * 1024), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds(ds, (lds_void*)(base + DK_DT + (wave * CPT + c) * 1024), 16, 0,
                                       0);
    }
    if (wave == 0 && lane < 32) {
      const float* ss = a.rst + (tile0 + tile) * (size_t)(2 * TR) + lane * 4;
      __builtin_amdgcn_global_load_lds(ss, (lds_void*)(smem + DK_STATS + stage * (2 * TR * 4)), 16, 0,
                                       0);
    }
  };

  int roff[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = 16 * rb + l16;
#pragma unroll
    for (int u = 0; u < 4; ++u) roff[rb][u] = row * 256 + (((4 * grp + u) ^ rswz(row)) << 4);
  }
  int toff[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) toff[st] = l16 * 128 + (((4 * st + grp) ^ tswz(l16)) << 4);
  // this lane's P slot of (st, kb) in the pair's hand-over buffer
  char* xp = smem + DKP_X + pair * (2 * 2 * 64 * 16) + lane * 16;
  // the row operand of S (Q, K waves) or dP (dO, V waves), and the
  // transposed operand of the row contraction (dO^T for dV, Q^T for dK)
  const int row_src = vwave ? DK_DR : DK_QR;
  const int t_src = vwave ? DK_QT : DK_DT;

  if (n_tiles > 0) issue(a.n_rt - 1, 0);
  auto step = [&](int u, auto stage_c, auto masked_c) {
    constexpr int STAGE_C = decltype(stage_c)::value;
    constexpr bool masked = decltype(masked_c)::value;
    const int stage = STAGE_C >= 0 ? STAGE_C : (u & 1);
    const int t = a.n_rt - 1 - u;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // the other stage held the previous tile, which every wave finished
    // reading before the barrier above
    if (u + 1 < n_tiles) issue(t - 1, stage ^ 1);
    const char* base = smem + stage * DK_STAGE;
    const char* stats = smem + DK_STATS + stage * (2 * TR * 4);

    // logits S (K waves) or dP (V waves) of the tile's 64 rows
    f32x4 x[2][2][KB];                                // [st][h2][kb]
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int rb = 2 * st + h2;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) x[st][h2][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const bf16x8 ra =
              *reinterpret_cast<const bf16x8*>(base + row_src + roff[rb & 1][uu] + (rb >> 1) * 8192);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) x[st][h2][kb] = OP::mma(ra, kv[kb].u[uu], x[st][h2][kb]);
        }
      }
    bf16x8 pk[2][KB];                                 // P (K waves) / dS (V waves), packed
    if (!vwave) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int rb = 2 * st + h2;
          const f32x4 l2v = *reinterpret_cast<const f32x4*>(stats + (16 * rb + 4 * grp) * 4);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float pv = fast_exp2(fmaf(x[st][h2][kb][e], a.c, -l2v[e]));
              if constexpr (masked) {
                const int pos = q_off + (t * TR + 16 * rb + 4 * grp + e) / G;
                if (jw + 16 * kb + l16 > pos) pv = 0.f;
              }
              pk[st][kb][4 * h2 + e] = (__bf16)pv;
            }
        }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          *reinterpret_cast<bf16x8*>(xp + (st * 2 + kb) * 1024) = pk[st][kb];
    }
    __syncthreads();                                  // P of every pair handed over
    if (vwave) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pv[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) pv[kb] = *reinterpret_cast<const bf16x8*>(xp + (st * 2 + kb) * 1024);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int rb = 2 * st + h2;
          const f32x4 dlv = *reinterpret_cast<const f32x4*>(stats + TR * 4 + (16 * rb + 4 * grp) * 4);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              pk[st][kb][4 * h2 + e] = (__bf16)((float)pv[kb][4 * h2 + e] * (x[st][h2][kb][e] - dlv[e]));
        }
      }
    }
    // dV^T += dOt . P (K waves) or dK^T += Qt . dS (V waves)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 ta = *reinterpret_cast<const bf16x8*>(base + t_src + toff[st] + db * 2048);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[kb][db] = OP::mma(ta, pk[st][kb], acc[kb][db]);
      }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int u = 0;
  for (; u + 1 < n_unm; u += 2) {
    step(u, S0{}, std::false_type{});
    step(u + 1, S1{}, std::false_type{});
  }
  if (u < n_unm) step(u++, S0{}, std::false_type{});
  for (; u < n_tiles; ++u) step(u, std::integral_constant<int, -1>{}, std::true_type{});

  // lane holds dV^T (K waves) or dK^T (V waves) at d = 16 db + 4 grp + e
  // for key jw + 16 kb + l16
  const float mul = vwave ? a.scale : 1.f;
  const void* add = vwave ? a.acc_k : a.acc_v;
  const float add_scale = add && a.acc_fixed ? a.acc_scale[vwave ? 2 : 3] : 0.f;
  __bf16* out = vwave ? a.dk : a.dv;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = jw + 16 * kb + l16;
    if (j >= a.n_kv) continue;
    const size_t off = ((size_t)b * a.n_kv + j) * kstride + (size_t)g * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      f32x4 xo = acc[kb][db] * mul;
      if (add && a.acc_fixed) {
        const long long* ap = static_cast<const long long*>(add) + off + 16 * db;
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[e] += (float)((double)ap[e] * add_scale);
      } else if (add) {
        xo += *reinterpret_cast<const f32x4*>(static_cast<const float*>(add) + off + 16 * db);
      }
      __attribute__((ext_vector_type(4))) __bf16 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)xo[e];
      *reinterpret_cast<decltype(w)*>(out + off + 16 * db) = w;
    }
  }
}

size_t bwd_rows_layout_tiles(const Shape& s) {
  const int G = s.h_q / s.h_kv;
  return (size_t)s.batch * s.h_kv * (((size_t)s.n_q * G + TR - 1) / TR);
}

hipError_t launch_bwd_rows_layout(const BwdPlan& p, hipStream_t st) {
  RowsArgs a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.dout = reinterpret_cast<const __bf16*>(p.dout);
  a.lse = p.lse; a.delta = p.delta;
  a.qt = reinterpret_cast<__bf16*>(p.qt);
  a.dot = reinterpret_cast<__bf16*>(p.dot);
  a.rst = p.rst;
  a.n_q = p.s.n_q; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  const int G = a.h_q / a.h_kv;
  a.n_rt = (int)(((size_t)a.n_q * G + TR - 1) / TR);
  hipLaunchKernelGGL(bwd_rows_layout_kernel, dim3((unsigned)bwd_rows_layout_tiles(p.s)), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdPlan& p, hipStream_t st) {
  DkdvArgs a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.dout = reinterpret_cast<const __bf16*>(p.dout);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.qt = reinterpret_cast<const __bf16*>(p.qt);
  a.dot = reinterpret_cast<const __bf16*>(p.dot);
  a.rst = p.rst;
  a.acc_k = p.acc_k; a.acc_v = p.acc_v; a.acc_fixed = p.acc_fixed; a.acc_scale = p.acc_scale;
  a.dk = reinterpret_cast<__bf16*>(p.dk);
  a.dv = reinterpret_cast<__bf16*>(p.dv);
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  const int G = a.h_q / a.h_kv;
  a.n_rt = (int)(((size_t)a.n_q * G + TR - 1) / TR);
  a.n_kt = (a.n_kv + DKP_KEYS - 1) / DKP_KEYS;
  a.q64 = TR / G; a.r64 = TR % G;
  a.scale = p.scale; a.c = p.s.scale_log2;
  struct DkdvLdsTag {};
  {
    const hipError_t e = ensure_dynamic_lds<DkdvLdsTag>(
        (const void*)attn_bwd_dkdv_bf16_pair_kernel, DKP_SMEM);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((size_t)a.n_kt * a.B * a.h_kv));
  hipLaunchKernelGGL(attn_bwd_dkdv_bf16_pair_kernel, grid, dim3(512), DKP_SMEM, st, a);
  return hipGetLastError();
}

}  // namespace hs2
