// Device-side helpers shared by the gfx950 kernels: the metadata view, vector
// types, MFMA wrappers, LDS swizzle and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "plan.hpp"

namespace ba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel-visible view of the plan metadata (pointers into the workspace).
struct Meta {
  const int32_t *group_heads;
  const QTile *qtiles;
  const int32_t *fwd_order;
  const int32_t *tile_row_id;
  const int32_t *tile_row_end;
  const int32_t *row_lo;
  const int32_t *row_hi;
  const int32_t *cu_branch;
  const int32_t *mode;
  const KTile *ktiles;
  const int32_t *bwd_order;
  int64_t N, Nq, Rb, A;
  int32_t hq, hkv, G, d, rows_per_tile;
  int32_t n_qtiles, n_ktiles;
  float scale;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap the two 32-lane halves of a wave: returns the value held by lane ^ 32.
__device__ __forceinline__ float half_swap(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// max / sum of a value over the two lanes l and l ^ 32.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int wave_min(int x) {
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

// LDS tiles of key rows (d bf16 each) are stored in 16-byte chunks whose index
// is XOR-swizzled by the row, so that both the row-wise 16-byte reads of the
// K operand and the 4-row transposed reads of the V operand spread over banks.
template <int HD>
__device__ __forceinline__ int swz(int row) {
  if constexpr (HD == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  else return ((row & 3) << 1) | ((row >> 2) & 1);
}
template <int HD>
__device__ __forceinline__ int lds_off(int row, int d) {  // element offset of (row, d)
  return row * HD + ((((d >> 3) ^ swz<HD>(row))) << 3) + (d & 7);
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// output lane i, slot j takes element (i % 4) of the 8 bytes addressed by input
// lane 4j + i/4.
__device__ __forceinline__ i16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace ba
