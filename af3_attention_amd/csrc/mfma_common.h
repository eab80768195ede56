// Shared device helpers for the bf16 MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "evoattn_internal.h"

namespace evo {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16 lane layout (checked on gfx950 hardware):
//   A[m][k]: lane l holds m = l % 32 and k = 8 * (l / 32) + i, i = 0..7
//   B[k][n]: lane l holds n = l % 32 and k = 8 * (l / 32) + i
//   D[m][n]: lane l, register v holds n = l % 32, m = 8 * (v / 4) + 4 * (l / 32) + v % 4
// Only the pairing of A's and B's k slots matters, so any permutation of the
// contraction index applied to both operands gives the same product.
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Row index (within a 32-row tile) of accumulator register v on lane l.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Two fp32 to packed bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Value of lane l ^ 32 combined with the own value: returns max over the pair.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t elem_offset(const Problem& p, int r, int pos, int h) {
  return ((static_cast<int64_t>(r) * p.row_stride + static_cast<int64_t>(pos) * p.pos_stride) * p.H + h) * p.D;
}

}  // namespace mfma

// Bias pre-pass shared by the MFMA kernels: out[h][j][k] (or out[h][k][j] when
// transpose_out) = sqrt(d) * bias[h][j][k] in fp32 over an np x np padded square;
// keys k >= N hold -inf and padded queries hold 0.
int bias_pad(int n);
hipError_t launch_bias_prep(const Problem& p, const void* bias, float* out, int np, int transpose_out,
                            hipStream_t s);

}  // namespace evo
