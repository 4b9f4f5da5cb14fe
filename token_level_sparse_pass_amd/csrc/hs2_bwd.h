// Device helpers shared by the backward-pass kernels: operands whose
// contraction index runs over rows or keys rather than the head dimension.
//
// An accumulator tile (hs2_device.h) gives lane l the values of indices
// 4*(l/16) + e, e = 0..3, of its 16-block; two such tiles cover 32 indices.
// Contracting over those 32 indices uses them in place: slot s of lane l
// stands for index slot_index(s, l/16). The other operand, X^T for a
// row-major X [index][D], is read with the head-dim rows permuted
// (d = DV * m + db, DV = D / 16, m = l % 16) so each lane loads one
// contiguous run of DV elements per index.
#pragma once

#include "hs2_device.h"

namespace hs2 {

// row slot s of a lane in the accumulator-shaped contraction order
__device__ __forceinline__ int slot_index(int s, int grp) {
  return s < 4 ? 4 * grp + s : 16 + 4 * grp + (s - 4);
}

// Transposed operand rows: raw[s][0..DV) = X[slot_index(s)][DV*(lane%16) ..]
template <typename T, int D>
struct TRows {
  static constexpr int DV = D / 16;
  T raw[8][DV];
};

template <typename T, int D>
__device__ __forceinline__ void load_trows(TRows<T, D>& t, const T* base, int ld, int lane) {
  constexpr int DV = D / 16;
  constexpr int BYTES = DV * sizeof(T);
  const int grp = lane >> 4;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const T* src = base + (size_t)slot_index(s, grp) * ld + DV * (lane & 15);
    if constexpr (BYTES == 16) {
      *reinterpret_cast<uint4*>(&t.raw[s][0]) = *reinterpret_cast<const uint4*>(src);
    } else if constexpr (BYTES == 8) {
      *reinterpret_cast<uint2*>(&t.raw[s][0]) = *reinterpret_cast<const uint2*>(src);
    } else {
#pragma unroll
      for (int e = 0; e < BYTES / 16; ++e)
        reinterpret_cast<uint4*>(&t.raw[s][0])[e] = reinterpret_cast<const uint4*>(src)[e];
    }
  }
}

// acc[db] += X^T(db) . Y over one 32-index contraction, where Y comes from
// two accumulator blocks y0 (indices 4*grp + e) and y1 (16 + 4*grp + e).
template <typename T, int D>
__device__ __forceinline__ void mma_t(f32x4 (&acc)[D / 16], const TRows<T, D>& x, const f32x4& y0,
                                      const f32x4& y1) {
  using OP = Op<T, D>;
  constexpr int DV = D / 16;
  if constexpr (sizeof(T) == 2) {
    bf16x8 yu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      yu[e] = (__bf16)y0[e];
      yu[4 + e] = (__bf16)y1[e];
    }
#pragma unroll
    for (int db = 0; db < DV; ++db) {
      bf16x8 xu;
#pragma unroll
      for (int s = 0; s < 8; ++s) xu[s] = x.raw[s][db];
      acc[db] = OP::mma(xu, yu, acc[db]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int db = 0; db < DV; ++db) {
        acc[db] = OP::mma(x.raw[e][db], y0[e], acc[db]);
        acc[db] = OP::mma(x.raw[4 + e][db], y1[e], acc[db]);
      }
  }
}

// The sparse layers' K/V sums that the full layer's dK/dV kernels add in:
// none, fp32, or 64-bit fixed point times `scale`.
struct AccIn {
  const void* base = nullptr;
  bool fixed = false;
  float scale = 0.f;
  __device__ __forceinline__ float at(size_t i) const {
    return fixed ? (float)((double)static_cast<const long long*>(base)[i] * scale)
                 : static_cast<const float*>(base)[i];
  }
};

// Store a transposed accumulator set (d = DV*(4*grp + e) + db) as row `dst`,
// times `mul`, plus the row of `add` that starts at element add_off (if any).
template <typename T, int D>
__device__ __forceinline__ void store_t_row(T* dst, const f32x4 (&acc)[D / 16], float mul,
                                            const AccIn& add, size_t add_off, int grp) {
  constexpr int DV = D / 16;
  T outv[4 * DV];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int db = 0; db < DV; ++db) {
      float x = acc[db][e] * mul;
      if (add.base) x += add.at(add_off + (4 * grp + e) * DV + db);
      outv[e * DV + db] = to_elem<T>(x);
    }
  constexpr int BYTES = 4 * DV * sizeof(T);
  uint4* out = reinterpret_cast<uint4*>(dst + grp * 4 * DV);
#pragma unroll
  for (int w = 0; w < BYTES / 16; ++w) out[w] = reinterpret_cast<uint4*>(outv)[w];
}


}  // namespace hs2
