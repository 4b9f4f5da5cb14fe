// Device-side building blocks shared by the gfx950 kernels of the Hybrid
// Block engine: operand types, the MFMA tile used everywhere, and small
// helpers. Every kernel is written for 64-lane wavefronts.
//
// The one MFMA shape used is a 16x16 output tile:
//   bf16:  v_mfma_f32_16x16x32_bf16  (8 operand elements per lane)
//   fp32:  v_mfma_f32_16x16x4_f32    (1 operand element per lane)
// Lane layout (checked on gfx950): lane l supplies A[row l%16][k-group l/16]
// and B[k-group l/16][col l%16]; it receives C[rows 4*(l/16) .. +3][col l%16].
//
// Dot products over the head dimension use a permuted k order: lane group
// q = l/16 owns the contiguous head-dim slice [q*D/4, (q+1)*D/4), and MFMA
// step s takes the s-th operand unit of that slice. A and B are loaded with
// the same rule, so the contraction is unchanged while every lane reads one
// contiguous D/4-element run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

template <typename T, int D>
struct Op;

template <int D>
struct Op<__bf16, D> {
  using unit = bf16x8;                      // one MFMA operand per lane
  static constexpr int ELEMS = 8;           // elements per unit
  static constexpr int SLICE = D / 4;       // elements per lane per row
  static constexpr int UNITS = SLICE / 8;   // MFMA steps over the head dim
  static __device__ __forceinline__ f32x4 mma(unit a, unit b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct Op<float, D> {
  using unit = float;
  static constexpr int ELEMS = 1;
  static constexpr int SLICE = D / 4;
  static constexpr int UNITS = SLICE;
  static __device__ __forceinline__ f32x4 mma(unit a, unit b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// A lane's head-dim slice of one row: SLICE elements, loaded as 16-byte words.
template <typename T, int D>
struct Frag {
  using O = Op<T, D>;
  typename O::unit u[O::UNITS];
};

template <typename T, int D>
__device__ __forceinline__ void load_slice(Frag<T, D>& f, const T* row, int lane) {
  // row points at element 0 of the row; the lane takes slice (lane/16)
  constexpr int BYTES = Op<T, D>::SLICE * sizeof(T);
  static_assert(BYTES % 16 == 0, "slice must be a multiple of 16 bytes");
  const uint4* src = reinterpret_cast<const uint4*>(row + (lane >> 4) * Op<T, D>::SLICE);
  uint4* dst = reinterpret_cast<uint4*>(&f.u[0]);
#pragma unroll
  for (int i = 0; i < BYTES / 16; ++i) dst[i] = src[i];
}

// The same operand with another k order, for rows gathered from global
// memory: lane group q takes the 16-byte chunks q, 4 + q, 8 + q, ... of the
// row, so the four lane groups of one load instruction read 64 contiguous
// bytes of each row (the per-lane slice above makes them read four pieces
// 64 bytes apart). A and B must be loaded with the same rule.
template <typename T, int D>
__device__ __forceinline__ void load_slice_il(Frag<T, D>& f, const T* row, int lane) {
  constexpr int BYTES = Op<T, D>::SLICE * sizeof(T);
  const uint4* src = reinterpret_cast<const uint4*>(row) + (lane >> 4);
  uint4* dst = reinterpret_cast<uint4*>(&f.u[0]);
#pragma unroll
  for (int m = 0; m < BYTES / 16; ++m) dst[m] = src[4 * m];
}

template <typename T, int D>
__device__ __forceinline__ void zero_slice(Frag<T, D>& f) {
  constexpr int BYTES = Op<T, D>::SLICE * sizeof(T);
  uint4* dst = reinterpret_cast<uint4*>(&f.u[0]);
#pragma unroll
  for (int i = 0; i < BYTES / 16; ++i) dst[i] = make_uint4(0, 0, 0, 0);
}

// acc += A_rows . B_rows^T over the head dim (A, B: one 16-row block each).
template <typename T, int D>
__device__ __forceinline__ f32x4 dot_tile(const Frag<T, D>& a, const Frag<T, D>& b, f32x4 acc) {
#pragma unroll
  for (int s = 0; s < Op<T, D>::UNITS; ++s) acc = Op<T, D>::mma(a.u[s], b.u[s], acc);
  return acc;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, WAVE));
}

// Maxima for kernels built with -fno-honor-nans (no operand quieting, so
// each is one max instruction; three-input maxima become v_max3_f32).
__device__ __forceinline__ float max2f(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
// max over the lanes l, l ^ 16, l ^ 32, l ^ 48: each gfx950 permlane swap
// hands a lane its partner row's value (16 lanes, then 32 lanes apart), with
// no LDS round trip
__device__ __forceinline__ float row_group_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2f(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2f(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Round-to-nearest-even store of an fp32 value in the tensor element type.
template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ float to_elem<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float x) { return (__bf16)x; }

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Work-group id remapped so that consecutive logical ids share an XCD (and
// therefore an L2): the dispatcher places work-group n on XCD n % 8.
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t bid, uint32_t nblocks) {
  const uint32_t nx = 8;
  const uint32_t per = nblocks / nx;           // full rounds
  const uint32_t tail = nblocks - per * nx;    // leftover ids stay in place
  if (bid >= per * nx) return bid;
  (void)tail;
  return (bid % nx) * per + bid / nx;
}


}  // namespace hs2
