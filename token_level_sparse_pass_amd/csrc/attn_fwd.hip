// Pass 1 of the full layer: causal grouped-query attention over the shared
// K/V cache (HySparse2 pages: openai-hub.net, section "From Hybrid SWA to
// HySparse2": the Full Attention layer produces the KV cache and decides
// which tokens matter; "Xiaomi Unveils HySparse2", section "Two-Level KV
// Sharing"). Besides O it records, for every (query, head), the softmax
// statistics m2 = max_j t_j and l = sum_j 2^(t_j - m2) with t = logit*log2(e),
// which the scoring pass needs to normalise probabilities exactly.
//
// Prefill: a work-group owns 128 "rows" of one (sequence, KV head g); a row
// is a (query, head-of-group) pair, so one K/V tile in LDS feeds all G query
// heads that share it. Four waves each hold two 16-row blocks.
// Decode (one query per sequence): each wave streams its own key range
// (split-KV), keeps every logit for the scoring step, and writes a partial
// (m2, l, O) record; a small kernel merges the records.
//
// MFMA mapping (hs2_device.h): logits^T = K . Q^T with K rows as A; then
// O^T += V^T . P^T with P taken straight from the logits accumulator. The
// head-dim rows of O^T are permuted (d = DV*m + db, DV = D/16) so that V is
// read as one contiguous DV-element run per key.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

struct FwdArgs {
  const void* q; const void* k; const void* v;
  void* o; float* stats; float* lse;
  int B, n_q, n_kv, h_q, h_kv, n_rt;
  float scale_log2;
};

constexpr float LN2 = 0.69314718055994530942f;

// Kahan-compensated running sum that is rescaled by alpha before each add.
struct KSum {
  float s, c;
  __device__ __forceinline__ void init() { s = 0.f; c = 0.f; }
  __device__ __forceinline__ void scale_add(float alpha, float x) {
    s *= alpha;
    c *= alpha;
    const float y = x - c;
    const float t = s + y;
    c = (t - s) - y;
    s = t;
  }
  __device__ __forceinline__ float value() const { return s - c; }
};

// V operands for one MFMA step, read from a row-major [key][D] tile.
// bf16: 8 key slots (k<4: base+4g+k, k>=4: base+16+4g+k-4) x DV values.
template <typename T, int D>
struct VRows {
  static constexpr int DV = D / 16;
  T raw[8][DV];
};

template <typename T, int D>
__device__ __forceinline__ void load_vrow(T* dst, const T* row, int lane) {
  constexpr int DV = D / 16;
  constexpr int BYTES = DV * sizeof(T);
  const T* src = row + DV * (lane & 15);
  if constexpr (BYTES == 16) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else if constexpr (BYTES == 8) {
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
  } else {
#pragma unroll
    for (int e = 0; e < BYTES / 16; ++e)
      reinterpret_cast<uint4*>(dst)[e] = reinterpret_cast<const uint4*>(src)[e];
  }
}

// ---------------------------------------------------------------------------
// prefill
// ---------------------------------------------------------------------------
template <typename T, int D>
struct FwdSmem {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LD = D + PAD;            // row stride in elements
  T k[2][64][LD];
  T v[2][64][LD];
};

template <typename T, int D, int RBW>
__global__ __launch_bounds__(256) void attn_fwd_prefill_kernel(FwdArgs a) {
  using OP = Op<T, D>;
  constexpr int DV = D / 16;
  constexpr int ROWS = 4 * RBW * 16;
  constexpr int VEC = 16 / sizeof(T);                 // elements per 16 B
  constexpr int V16_ROW = D / VEC;                    // 16-byte words per row
  constexpr int LOADS = 64 * V16_ROW / 256;           // per thread per tensor
  __shared__ FwdSmem<T, D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int G = a.h_q / a.h_kv;
  const int R = a.n_q * G;
  const int q_off = a.n_kv - a.n_q;

  // longest first over the whole grid (row tile descending, every
  // (sequence, KV head) at each step): balances causal work
  const int rt = a.n_rt - 1 - (int)(blockIdx.x / (a.B * a.h_kv));
  const int bg = blockIdx.x % (a.B * a.h_kv);
  const int b = bg % a.B;
  const int g = bg / a.B;
  const int r0 = rt * ROWS;
  const int i_hi = min(a.n_q - 1, (r0 + ROWS - 1) / G);
  const int p_hi = q_off + i_hi;
  const int n_tiles = (p_hi + 64) / 64;

  const T* qb = reinterpret_cast<const T*>(a.q);
  const T* kseq = reinterpret_cast<const T*>(a.k) + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const T* vseq = reinterpret_cast<const T*>(a.v) + ((size_t)b * a.n_kv * a.h_kv + g) * D;
  const size_t kstride = (size_t)a.h_kv * D;

  Frag<T, D> qf[RBW];
  int row_pos[RBW];                                    // causal limit per row
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int r = r0 + wave * RBW * 16 + rb * 16 + (lane & 15);
    if (r < R) {
      const int i = r / G, hh = r - (r / G) * G;
      load_slice<T, D>(qf[rb], qb + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D, lane);
      row_pos[rb] = q_off + i;
    } else {
      zero_slice<T, D>(qf[rb]);
      row_pos[rb] = -1;
    }
  }

  float m_run[RBW];
  KSum l_run[RBW];
  f32x4 acc[RBW][DV];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb].init();
#pragma unroll
    for (int db = 0; db < DV; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int tile) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + 256 * it;
      const int row = u / V16_ROW, c16 = u - (u / V16_ROW) * V16_ROW;
      const int j = tile * 64 + row;
      if (j < a.n_kv) {
        kreg[it] = *reinterpret_cast<const uint4*>(kseq + (size_t)j * kstride + c16 * VEC);
        vreg[it] = *reinterpret_cast<const uint4*>(vseq + (size_t)j * kstride + c16 * VEC);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int u = threadIdx.x + 256 * it;
      const int row = u / V16_ROW, c16 = u - (u / V16_ROW) * V16_ROW;
      *reinterpret_cast<uint4*>(&sm.k[buf][row][c16 * VEC]) = kreg[it];
      *reinterpret_cast<uint4*>(&sm.v[buf][row][c16 * VEC]) = vreg[it];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) gload(t + 1);
    const int j0 = t * 64;

    f32x4 s[RBW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<T, D> kf;
      load_slice<T, D>(kf, &sm.k[buf][kb * 16 + (lane & 15)][0], lane);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        s[rb][kb] = dot_tile<T, D>(kf, qf[rb], f32x4{0.f, 0.f, 0.f, 0.f});
    }

    const bool need_mask = (j0 + 63) > (q_off + r0 / G);
    float p[RBW][16];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = s[rb][kb][e] * a.scale_log2;
          if (need_mask && (j0 + kb * 16 + 4 * grp + e) > row_pos[rb]) x = -INFINITY;
          p[rb][kb * 4 + e] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = xor_max(tmax, 16);
      tmax = xor_max(tmax, 32);
      const float m_new = fmaxf(m_run[rb], tmax);
      const float alpha = fast_exp2(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[rb][e] = fast_exp2(p[rb][e] - m_new);
        psum += p[rb][e];
      }
      l_run[rb].scale_add(alpha, psum);
#pragma unroll
      for (int db = 0; db < DV; ++db) acc[rb][db] *= alpha;
    }

    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        VRows<T, D> vr;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int key = st * 32 + (sl < 4 ? 4 * grp + sl : 16 + 4 * grp + sl - 4);
          load_vrow<T, D>(&vr.raw[sl][0], &sm.v[buf][key][0], lane);
        }
        bf16x8 pu[RBW];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
          for (int e = 0; e < 8; ++e) pu[rb][e] = (__bf16)p[rb][st * 8 + e];
#pragma unroll
        for (int db = 0; db < DV; ++db) {
          bf16x8 vu;
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) vu[sl] = vr.raw[sl][db];
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) acc[rb][db] = OP::mma(vu, pu[rb], acc[rb][db]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          T vv[DV];
          load_vrow<T, D>(vv, &sm.v[buf][kb * 16 + 4 * grp + e][0], lane);
#pragma unroll
          for (int db = 0; db < DV; ++db)
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
              acc[rb][db] = OP::mma(vv[db], p[rb][kb * 4 + e], acc[rb][db]);
        }
    }

    if (t + 1 < n_tiles) sstore(buf ^ 1);
    __syncthreads();
  }

  T* ob = reinterpret_cast<T*>(a.o);
  const size_t plane = (size_t)a.B * a.h_q * a.n_q;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    float l = l_run[rb].value();
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = r0 + wave * RBW * 16 + rb * 16 + (lane & 15);
    if (r >= R) continue;
    const int i = r / G, hh = r - (r / G) * G;
    const int h = g * G + hh;
    const float inv = 1.f / l;
    T outv[4 * DV];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int db = 0; db < DV; ++db) outv[e * DV + db] = to_elem<T>(acc[rb][db][e] * inv);
    T* orow = ob + (((size_t)b * a.n_q + i) * a.h_q + h) * D + grp * 4 * DV;
#pragma unroll
    for (int w = 0; w < (int)(4 * DV * sizeof(T)) / 16; ++w)
      reinterpret_cast<uint4*>(orow)[w] = reinterpret_cast<uint4*>(outv)[w];
    if (grp == 0) {
      const size_t si = ((size_t)b * a.h_q + h) * a.n_q + i;
      a.stats[si] = m_run[rb];
      a.stats[plane + si] = l;
      a.stats[2 * plane + si] = 1.f / l;
      if (a.lse) a.lse[si] = (m_run[rb] + log2f(l)) * LN2;
    }
  }
}

template <typename T, int D>
static hipError_t launch_prefill_t(const FwdPlan& p, hipStream_t st) {
  constexpr int RBW = 2;
  constexpr int ROWS = 4 * RBW * 16;
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.stats = p.stats; a.lse = p.lse;
  a.B = p.s.batch; a.n_q = p.s.n_q; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.scale_log2 = p.s.scale_log2;
  const int G = a.h_q / a.h_kv;
  a.n_rt = (a.n_q * G + ROWS - 1) / ROWS;
  const dim3 grid((unsigned)((size_t)a.n_rt * a.B * a.h_kv));
  hipLaunchKernelGGL((attn_fwd_prefill_kernel<T, D, RBW>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_prefill_generic(const FwdPlan& p, hipStream_t st) {
  if (p.s.bf16) {
    if (p.s.head_dim == 128) return launch_prefill_t<__bf16, 128>(p, st);
    if (p.s.head_dim == 64) return launch_prefill_t<__bf16, 64>(p, st);
  } else {
    if (p.s.head_dim == 128) return launch_prefill_t<float, 128>(p, st);
    if (p.s.head_dim == 64) return launch_prefill_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// decode: split-KV with stored logits
// ---------------------------------------------------------------------------
struct DecArgs {
  const void* q; const void* k; const void* v;
  float* part; float* logits; size_t lstride;
  const int32_t* seq_len;
  KvRows kv;
  int B, n_kv, h_q, h_kv, kps, n_split;
  float scale_log2;
};

template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void attn_fwd_decode_kernel(DecArgs a) {
  using OP = Op<T, D>;
  constexpr int DV = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int G = a.h_q / a.h_kv;
  const int wg_per_bg = a.n_split / 4;
  const int bg = blockIdx.x / wg_per_bg;
  const int split = (blockIdx.x - bg * wg_per_bg) * 4 + wave;
  const int b = bg / a.h_kv;
  const int g = bg - b * a.h_kv;
  const int n_keys = a.seq_len ? a.seq_len[b] : a.n_kv;   // keys of this sequence
  const int k_begin = split * a.kps;
  const int k_end = min(n_keys, k_begin + a.kps);

  const T* qb = reinterpret_cast<const T*>(a.q);
  // K/V rows of key j: kseq + kv.row(b, j) * kstride (contiguous or paged)
  const T* kseq = reinterpret_cast<const T*>(a.k) + (size_t)g * D;
  const T* vseq = reinterpret_cast<const T*>(a.v) + (size_t)g * D;
  const size_t kstride = (size_t)a.h_kv * D;

  Frag<T, D> qf[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int hh = rb * 16 + (lane & 15);
    if (hh < G) load_slice<T, D>(qf[rb], qb + ((size_t)b * a.h_q + g * G + hh) * D, lane);
    else zero_slice<T, D>(qf[rb]);
  }
  float m_run[RB];
  KSum l_run[RB];
  f32x4 acc[RB][DV];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb].init();
#pragma unroll
    for (int db = 0; db < DV; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int j0 = k_begin; j0 < k_end; j0 += 64) {
    Frag<T, D> kf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int j = j0 + kb * 16 + (lane & 15);
      if (j < k_end) load_slice<T, D>(kf[kb], kseq + a.kv.row(b, j) * kstride, lane);
      else zero_slice<T, D>(kf[kb]);
    }
    // V rows for the lane's slots: st-th 32-key step, slot sl
    T vraw[2][8][DV];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const int j = j0 + st * 32 + (sl < 4 ? 4 * grp + sl : 16 + 4 * grp + sl - 4);
        load_vrow<T, D>(&vraw[st][sl][0], vseq + a.kv.row(b, j < k_end ? j : k_begin) * kstride,
                        lane);
      }

    float p[RB][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4 sv = dot_tile<T, D>(kf[kb], qf[rb], f32x4{0.f, 0.f, 0.f, 0.f});
        float xs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + kb * 16 + 4 * grp + e;
          float x = sv[e] * a.scale_log2;
          xs[e] = sv[e];
          if (j >= k_end) x = -INFINITY;
          p[rb][kb * 4 + e] = x;
          tmax = fmaxf(tmax, x);
        }
        // keep the raw logits (q.k) of valid heads for the scoring step
        const int hh = rb * 16 + (lane & 15);
        if (hh < G) {
          float* lg = a.logits + ((size_t)b * a.h_q + g * G + hh) * a.lstride;
          const int jb = j0 + kb * 16 + 4 * grp;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (jb + e < k_end) lg[jb + e] = xs[e];
        }
      }
      tmax = xor_max(tmax, 16);
      tmax = xor_max(tmax, 32);
      const float m_new = fmaxf(m_run[rb], tmax);
      const float alpha = fast_exp2(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[rb][e] = fast_exp2(p[rb][e] - m_new);
        psum += p[rb][e];
      }
      l_run[rb].scale_add(alpha, psum);
#pragma unroll
      for (int db = 0; db < DV; ++db) acc[rb][db] *= alpha;
    }

    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 pu[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int e = 0; e < 8; ++e) pu[rb][e] = (__bf16)p[rb][st * 8 + e];
#pragma unroll
        for (int db = 0; db < DV; ++db) {
          bf16x8 vu;
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) vu[sl] = vraw[st][sl][db];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) acc[rb][db] = OP::mma(vu, pu[rb], acc[rb][db]);
        }
      }
    } else {
      // fp32: slot (st, sl) holds key st*32 + (kb-local) with kb = 2*st + sl/4
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
#pragma unroll
          for (int db = 0; db < DV; ++db)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[rb][db] = OP::mma(to_f32(vraw[st][sl][db]), p[rb][st * 8 + sl], acc[rb][db]);
    }
  }

  // partial record per (b, head, split): m2, l, O[D] (unnormalised)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l = l_run[rb].value();
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int hh = rb * 16 + (lane & 15);
    if (hh >= G) continue;
    float* rec = a.part + (((size_t)b * a.h_q + g * G + hh) * a.n_split + split) * (D + 2);
    if (grp == 0) {
      rec[0] = m_run[rb];
      rec[1] = l;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int db = 0; db < DV; ++db) rec[2 + DV * (4 * grp + e) + db] = acc[rb][db][e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* part, int n_split, T* o,
                                                           float* stats, float* lse, size_t plane) {
  // one work-group per (b, head); thread d owns output element d. The
  // splits' maxima, weights 2^(m_s - M) and row sums are read by all
  // threads together into LDS, a chunk of splits at a time, so each thread's
  // loop over splits only loads its own element of every split (loads that
  // do not depend on one another); the sums still run in split order.
  constexpr int CH = 512;
  __shared__ float w_sh[CH], l_sh[CH], red[D / 64];
  const size_t bh = blockIdx.x;
  const float* rec = part + bh * n_split * (D + 2);
  const int d = threadIdx.x;
  float M = -1e30f;
  for (int s = d; s < n_split; s += D) M = fmaxf(M, rec[(size_t)s * (D + 2)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if ((d & 63) == 0) red[d >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < D / 64; ++i) M = fmaxf(M, red[i]);
  float L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += CH) {
    const int n = min(CH, n_split - s0);
    __syncthreads();                              // the previous chunk's weights are used
    for (int s = d; s < n; s += D) {
      const float* r = rec + (size_t)(s0 + s) * (D + 2);
      w_sh[s] = fast_exp2(r[0] - M);
      l_sh[s] = r[1];
    }
    __syncthreads();
    const float* r = rec + (size_t)s0 * (D + 2) + 2 + d;
#pragma unroll 8
    for (int s = 0; s < n; ++s) acc += r[(size_t)s * (D + 2)] * w_sh[s];
    // every thread forms the same L from the broadcast LDS values
    for (int s = 0; s < n; ++s) L += l_sh[s] * w_sh[s];
  }
  o[bh * D + d] = to_elem<T>(acc / L);
  if (d == 0) {
    stats[bh] = M;
    stats[plane + bh] = L;
    stats[2 * plane + bh] = 1.f / L;
    if (lse) lse[bh] = (M + log2f(L)) * LN2;
  }
}

int decode_n_split(int n_kv, int* keys_per_split) {
  // about 2048 keys per wave; whole 64-key tiles; a multiple of 4 waves
  int kps = 2048;
  int n = (n_kv + kps - 1) / kps;
  n = (n + 3) / 4 * 4;
  kps = ((n_kv + n - 1) / n + 63) / 64 * 64;
  *keys_per_split = kps;
  return n;
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodePlan& p, hipStream_t st) {
  DecArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.part = p.part; a.logits = p.logits;
  a.lstride = p.logits_stride; a.seq_len = p.seq_len; a.kv = p.kv;
  a.B = p.s.batch; a.n_kv = p.s.n_kv; a.h_q = p.s.h_q; a.h_kv = p.s.h_kv;
  a.kps = p.keys_per_split; a.n_split = p.n_split; a.scale_log2 = p.s.scale_log2;
  const int G = a.h_q / a.h_kv;
  const dim3 grid((unsigned)((size_t)a.B * a.h_kv * (a.n_split / 4)));
  hipError_t e;
  if (decode_uses_bf16_kernel(p.s)) {
    e = launch_attn_decode_bf16(p, st);
  } else {
    if (G <= 16) hipLaunchKernelGGL((attn_fwd_decode_kernel<T, D, 1>), grid, dim3(256), 0, st, a);
    else if (G <= 32) hipLaunchKernelGGL((attn_fwd_decode_kernel<T, D, 2>), grid, dim3(256), 0, st, a);
    else return hipErrorInvalidValue;
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const size_t plane = (size_t)a.B * a.h_q;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)plane), dim3(D), 0, st,
                     p.part, p.n_split, reinterpret_cast<T*>(p.o), p.stats, p.lse, plane);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_decode(const DecodePlan& p, hipStream_t st) {
  if (p.s.bf16) {
    if (p.s.head_dim == 128) return launch_decode_t<__bf16, 128>(p, st);
    if (p.s.head_dim == 64) return launch_decode_t<__bf16, 64>(p, st);
  } else {
    if (p.s.head_dim == 128) return launch_decode_t<float, 128>(p, st);
    if (p.s.head_dim == 64) return launch_decode_t<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

// S[b][j] = sum over heads (in order) of 2^(c * logit - m2) / l, candidates only.
// Logits are one row per (sequence, query head), so each head's read is
// contiguous across the threads of a block.
__global__ __launch_bounds__(256) void decode_score_kernel(DecodeScorePlan a) {
  extern __shared__ float sh[];                  // m2[h_q], inv_l[h_q]
  const int b = blockIdx.y;
  const size_t plane = (size_t)a.batch * a.h_q;
  for (int h = threadIdx.x; h < a.h_q; h += blockDim.x) {
    sh[h] = a.stats[(size_t)b * a.h_q + h];
    sh[a.h_q + h] = a.stats[2 * plane + (size_t)b * a.h_q + h];
  }
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int n_cand = a.seq_len ? a.seq_len[b] - a.window : a.n_cand;
  if (j >= n_cand) return;
  const float* lg = a.logits + (size_t)b * a.h_q * a.logits_stride + j;
  float s = 0.f;
  for (int h = 0; h < a.h_q; ++h)
    // each logit is read once: non-temporal loads
    s = fmaf(fast_exp2(fmaf(__builtin_nontemporal_load(lg + (size_t)h * a.logits_stride), a.c, -sh[h])),
             sh[a.h_q + h], s);
  a.scores[(size_t)b * a.score_stride + j] = s;
}

hipError_t launch_decode_score(const DecodeScorePlan& p, hipStream_t st) {
  if (p.n_cand <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.n_cand + 255) / 256), (unsigned)p.batch);
  hipLaunchKernelGGL(decode_score_kernel, grid, dim3(256), 2 * p.h_q * sizeof(float), st, p);
  return hipGetLastError();
}

}  // namespace hs2
