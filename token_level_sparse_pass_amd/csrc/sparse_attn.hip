// Sparse attention with KV Reuse: every sparse layer of a Hybrid Block
// attends, with one softmax, over the same index set (window + selected
// tokens) and reads the same K/V as the full layer (HySparse2 pages: "Xiaomi
// Unveils HySparse2 for Faster Long-Context AI", sections "Two-Level KV
// Sharing" and "Token-Level Selection and Unified Local Access").
//
// One work-group serves one (sequence b, query i, KV head g). Its rows are
// all (layer, query head of group g) pairs, so each selected K/V row is
// gathered from HBM once and used by G heads x L layers. The index list is
// walked in tiles of 32 keys; NW waves split the list and merge their
// online-softmax states through LDS at the end (NW > 1 serves few queries,
// as in decode, where the bf16 head-dim-128 kernels do not apply).
//
// Per 32-key tile, in MFMA terms (16x16 tiles, see hs2_device.h):
//   logits^T (keys x rows) = K_sel . Q^T        A = gathered K rows, B = Q rows
//   O^T (head-dim x rows) += V_sel^T . P^T      A = gathered V, B = P in regs
// P^T comes straight out of the logits accumulator (lane l holds row l%16 and
// keys 4*(l/16)+i of each 16-key block), so the key order of the second
// product follows that layout. The head-dim rows of O^T are permuted so that
// lane l needs V[key][DV*(l%16) .. +DV-1], DV = D/16: one contiguous load per
// key; for bf16 an in-register 8x8 transpose turns those into MFMA operands.
#include "hs2_device.h"
#include "hs2_launch.h"

namespace hs2 {

struct SparseArgs {
  const void* q;        // [L, B, n_q, h_q, D]
  const void* k;        // [B, n_kv, h_kv, D]
  const void* v;
  const int32_t* idx;   // [B, n_q, W]
  void* o;              // [L, B, n_q, h_q, D]
  int L, B, n_q, n_kv, h_q, h_kv, W;
  float scale_log2;     // softmax scale * log2(e)
  KvRows kv;            // key j of sequence b is K/V buffer row kv.row(b, j)
  size_t layer_stride;  // elements between layers of q and o
};

template <typename T, int D>
struct VTile {
  static constexpr int DV = D / 16;                 // head-dim values per lane
  // raw[k]: lane's DV values of key slot k (k<4: 4g+k, k>=4: 16+4g+k-4)
  T raw[8][DV];
};

template <typename T, int D>
__device__ __forceinline__ void load_v_rows(VTile<T, D>& vt, const T* vbase, const size_t* key_off,
                                            int lane) {
  constexpr int DV = D / 16;
  constexpr int BYTES = DV * sizeof(T);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const T* row = vbase + (size_t)key_off[s] + DV * (lane & 15);
    if constexpr (BYTES == 16) {
      *reinterpret_cast<uint4*>(&vt.raw[s][0]) = *reinterpret_cast<const uint4*>(row);
    } else if constexpr (BYTES == 8) {
      *reinterpret_cast<uint2*>(&vt.raw[s][0]) = *reinterpret_cast<const uint2*>(row);
    } else {
#pragma unroll
      for (int e = 0; e < BYTES / 16; ++e)
        reinterpret_cast<uint4*>(&vt.raw[s][0])[e] = reinterpret_cast<const uint4*>(row)[e];
    }
  }
}

template <typename T, int D, int RB, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_kernel(SparseArgs a) {
  using OP = Op<T, D>;
  constexpr int DV = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.h_q / a.h_kv;
  const int rows_total = a.L * G;

  const uint32_t wg = xcd_swizzle(blockIdx.x, gridDim.x);
  const int g = wg % a.h_kv;
  const int bi = wg / a.h_kv;              // b * n_q + i
  const int b = bi / a.n_q;
  const int i = bi - b * a.n_q;

  const T* qb = reinterpret_cast<const T*>(a.q);
  const T* kb = reinterpret_cast<const T*>(a.k);
  const T* vb = reinterpret_cast<const T*>(a.v);
  const int32_t* irow = a.idx + (size_t)bi * a.W;

  // Q fragments (B operand): row r = layer * G + hh
  Frag<T, D> qf[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + (lane & 15);
    if (r < rows_total) {
      const int layer = r / G, hh = r - (r / G) * G;
      const T* qrow = qb + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D);
      load_slice_il<T, D>(qf[rb], qrow, lane);
    } else {
      zero_slice<T, D>(qf[rb]);
    }
  }

  // Split kernel: the index row is staged in LDS once, so a tile's gathers
  // do not wait on a global index load first.
  constexpr int IDX_LDS = NW > 1 ? 4096 : 1;
  __shared__ int s_idx[IDX_LDS];
  if constexpr (NW > 1) {
    for (int x = threadIdx.x; x < min(a.W, IDX_LDS); x += 64 * NW) s_idx[x] = irow[x];
    __syncthreads();
  }
  auto idx_at = [&](int pos) -> int {
    if constexpr (NW > 1) return pos < IDX_LDS ? s_idx[pos] : irow[pos];
    return irow[pos];
  };

  // number of valid indices: rows are a valid prefix followed by -1
  int n_valid = 0;
  for (int t = lane; t < a.W; t += 64) n_valid += (idx_at(t) >= 0) ? 1 : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n_valid += __shfl_xor(n_valid, m, 64);

  // this wave's share of the index list, in whole 32-key tiles
  const int n_tiles = (n_valid + 31) / 32;
  const int t_begin = (n_tiles * wave) / NW;
  const int t_end = (n_tiles * (wave + 1)) / NW;

  float m_run[RB], l_run[RB];
  f32x4 acc[RB][DV];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DV; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_row_stride = (size_t)a.h_kv * D;      // elements between buffer rows
  const T* kseq = kb + (size_t)g * D;                   // + buffer row * kv_row_stride
  const T* vseq = vb + (size_t)g * D;
  const int grp = lane >> 4;

  // one 32-key tile's K rows (key slot 16*kb + lane%16) and V rows (this
  // lane's 8 key slots)
  struct TileRegs {
    Frag<T, D> kf[2];
    VTile<T, D> vt;
  };
  auto fetch = [&](int t, TileRegs& r) {
    const int base = t * 32;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int pos = base + kb2 * 16 + (lane & 15);
      const int j = pos < n_valid ? idx_at(pos) : 0;
      load_slice_il<T, D>(r.kf[kb2], kseq + a.kv.row(b, j) * kv_row_stride, lane);
    }
    size_t voff[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int pos = base + (s < 4 ? 4 * grp + s : 16 + 4 * grp + (s - 4));
      voff[s] = a.kv.row(b, pos < n_valid ? idx_at(pos) : 0) * kv_row_stride;
    }
    load_v_rows<T, D>(r.vt, vseq, voff, lane);
  };

  auto compute = [&](int t, const TileRegs& r) {
    const int base = t * 32;
    const Frag<T, D>(&kf)[2] = r.kf;
    const VTile<T, D>& vt = r.vt;

    // logits and online softmax per row block
    typename OP::unit pu[RB][(sizeof(T) == 2) ? 1 : 8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = dot_tile<T, D>(kf[kb2], qf[rb], f32x4{0.f, 0.f, 0.f, 0.f});
      }
      // lane's keys: slot (kb2, e) -> tile key 16*kb2 + 4*grp + e
      float tmax = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = (base + 16 * kb2 + 4 * grp + e) < n_valid;
          float x = ok ? s[kb2][e] * a.scale_log2 : -INFINITY;
          s[kb2][e] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = xor_max(tmax, 16);
      tmax = xor_max(tmax, 32);
      const float m_new = fmaxf(m_run[rb], tmax);
      const float alpha = fast_exp2(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float psum = 0.f;
      float p[8];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(s[kb2][e] - m_new);
          p[kb2 * 4 + e] = pe;
          psum += pe;
        }
      l_run[rb] = l_run[rb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DV; ++db) acc[rb][db] *= alpha;
      if constexpr (sizeof(T) == 2) {
        bf16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = (__bf16)p[e];
        pu[rb][0] = u;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pu[rb][e] = p[e];
      }
    }

    // O^T += V^T . P^T
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int db = 0; db < DV; ++db) {
        bf16x8 vu;
#pragma unroll
        for (int s = 0; s < 8; ++s) vu[s] = vt.raw[s][db];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][db] = OP::mma(vu, pu[rb][0], acc[rb][db]);
      }
    } else {
      // fp32: one MFMA per (key slot): k-group grp covers slot keys
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int db = 0; db < DV; ++db)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][db] = OP::mma(to_f32(vt.raw[s][db]), pu[rb][s], acc[rb][db]);
    }
  };

  for (int t = t_begin; t < t_end; ++t) {
    TileRegs tr;
    fetch(t, tr);
    compute(t, tr);
  }

  // row totals over the 4 lanes that share a row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16, 64);
    l_run[rb] += __shfl_xor(l_run[rb], 32, 64);
  }

  T* ob = reinterpret_cast<T*>(a.o);
  if constexpr (NW == 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + (lane & 15);
      if (r >= rows_total) continue;
      const int layer = r / G, hh = r - (r / G) * G;
      T* orow = ob + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D);
      const float inv = l_run[rb] > 0.f ? 1.f / l_run[rb] : 0.f;
      T outv[4 * DV];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int db = 0; db < DV; ++db) outv[e * DV + db] = to_elem<T>(acc[rb][db][e] * inv);
      constexpr int BYTES = 4 * DV * sizeof(T);
      uint4* dst = reinterpret_cast<uint4*>(orow + grp * 4 * DV);
#pragma unroll
      for (int w = 0; w < BYTES / 16; ++w) dst[w] = reinterpret_cast<uint4*>(outv)[w];
    }
  } else {
    // merge the NW partial states through LDS, one row block at a time
    __shared__ float sm_m[NW][64];
    __shared__ float sm_l[NW][64];
    __shared__ float sm_o[NW][16][D + 1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (grp == 0) {
        sm_m[wave][rb * 16 + lane] = m_run[rb];
        sm_l[wave][rb * 16 + lane] = l_run[rb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rr = rb * 16 + (lane & 15);
      float M = -1e30f;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][rr]);
      const float sc = fast_exp2(m_run[rb] - M);
      // this wave's O block, rescaled, into LDS
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int db = 0; db < DV; ++db)
          sm_o[wave][lane & 15][DV * (4 * grp + e) + db] = acc[rb][db][e] * sc;
      __syncthreads();
      // every thread finishes some (row, d) outputs, summing waves in order
      for (int x = threadIdx.x; x < 16 * D; x += 64 * NW) {
        const int row = x / D, d = x - (x / D) * D;
        const int r = rb * 16 + row;
        if (r < rows_total) {
          float Mr = -1e30f;
          for (int w = 0; w < NW; ++w) Mr = fmaxf(Mr, sm_m[w][r]);
          float Lr = 0.f, o = 0.f;
          for (int w = 0; w < NW; ++w) {
            Lr += sm_l[w][r] * fast_exp2(sm_m[w][r] - Mr);
            o += sm_o[w][row][d];
          }
          const int layer = r / G, hh = r - (r / G) * G;
          T* orow = ob + ((size_t)layer * a.layer_stride + (((size_t)b * a.n_q + i) * a.h_q + g * G + hh) * D);
          orow[d] = to_elem<T>(Lr > 0.f ? o / Lr : 0.f);
        }
      }
      __syncthreads();
    }
  }
}

template <typename T, int D, int NW>
static hipError_t launch_sparse_rb(const SparseArgs& a, int rb, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)a.B * a.n_q * a.h_kv));
  const dim3 block(64 * NW);
  switch (rb) {
    case 1: hipLaunchKernelGGL((sparse_attn_kernel<T, D, 1, NW>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((sparse_attn_kernel<T, D, 2, NW>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((sparse_attn_kernel<T, D, 3, NW>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((sparse_attn_kernel<T, D, 4, NW>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_sparse_t(const SparseArgs& a, int rb, bool split, hipStream_t st) {
  return split ? launch_sparse_rb<T, D, 8>(a, rb, st) : launch_sparse_rb<T, D, 1>(a, rb, st);
}

bool sparse_uses_bf16_kernel(const SparsePlan& p);
hipError_t launch_sparse_attn_bf16(const SparsePlan& p, hipStream_t st);
bool sparse_uses_bf16_split_kernel(const SparsePlan& p);
hipError_t launch_sparse_attn_bf16_split(const SparsePlan& p, hipStream_t st);

hipError_t launch_sparse_attn(const SparsePlan& p, hipStream_t st) {
  if (sparse_uses_bf16_kernel(p)) return launch_sparse_attn_bf16(p, st);
  if (sparse_uses_bf16_split_kernel(p)) return launch_sparse_attn_bf16_split(p, st);
  SparseArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.idx = p.idx; a.o = p.o;
  a.L = p.layers; a.B = p.batch; a.n_q = p.n_q; a.n_kv = p.n_kv;
  a.h_q = p.h_q; a.h_kv = p.h_kv; a.W = p.width; a.scale_log2 = p.scale_log2; a.kv = p.kv;
  a.layer_stride = p.layer_stride ? p.layer_stride
                                  : (size_t)p.batch * p.n_q * p.h_q * p.head_dim;
  const int G = p.h_q / p.h_kv;
  const int rb = (p.layers * G + 15) / 16;
  // few work-groups: split each index list over 8 waves of one work-group
  const bool split = (size_t)p.batch * p.n_q * p.h_kv < 2048;
  if (p.bf16) {
    if (p.head_dim == 128) return launch_sparse_t<__bf16, 128>(a, rb, split, st);
    if (p.head_dim == 64) return launch_sparse_t<__bf16, 64>(a, rb, split, st);
  } else {
    if (p.head_dim == 128) return launch_sparse_t<float, 128>(a, rb, split, st);
    if (p.head_dim == 64) return launch_sparse_t<float, 64>(a, rb, split, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hs2
