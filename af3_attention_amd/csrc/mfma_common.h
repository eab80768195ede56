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
typedef short i16x4 __attribute__((ext_vector_type(4)));

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

// max(a, b, c); the compiler fuses it into one v_max3_f32.  (Not inline asm: the
// compiler's hazard checks do not see which registers an asm statement reads, so
// an asm read of a fresh MFMA result could miss the required wait states.)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ int64_t elem_offset(const Problem& p, int r, int pos, int h) {
  return ((static_cast<int64_t>(r) * p.row_stride + static_cast<int64_t>(pos) * p.pos_stride) * p.H + h) * p.D;
}

// Element offset of (r, 0, h, 0): the start of the (row, head) slab.
__device__ __forceinline__ int64_t row_head_offset(const Problem& p, int r, int h) {
  return (static_cast<int64_t>(r) * p.row_stride * p.H + h) * p.D;
}

template <int D>
struct Shape {
  static constexpr int KS = D >= 16 ? D / 16 : 1;  // 16-deep MFMA steps over d
  static constexpr int DB = D >= 32 ? D / 32 : 1;  // 32-row blocks over d for transposed outputs
};

// MFMA operand straight from global memory: position pos (the lane's row or
// column), d = 16 ks + 8 half + i.  Zero outside the tensor.
template <int D>
__device__ __forceinline__ u32x4 global_operand(const Problem& p, const uint16_t* src, int r, int pos, int h, int ks,
                                                int half) {
  const int d0 = ks * 16 + 8 * half;
  if (pos >= p.N || d0 >= D) return u32x4{0u, 0u, 0u, 0u};
  typedef __attribute__((address_space(1))) const u32x4 gu32x4;  // a global (not flat) load
  return *(gu32x4*)(src + elem_offset(p, r, pos, h) + d0);
}

// Store a transposed [d][pos] accumulator (lane = position) as bf16 into the
// [d] row of one position, times `scale`.
template <int D>
__device__ __forceinline__ void store_dT(uint16_t* dst_row, const f32x16* acc, float scale, int half) {
#pragma unroll
  for (int db = 0; db < Shape<D>::DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * half;
      if (d < D) {
        const u32x2 w = {pack_bf16(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale),
                         pack_bf16(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale)};
        *reinterpret_cast<u32x2*>(dst_row + d) = w;
      }
    }
  }
}

// The same store with 16-byte pieces (d = 16, 32): lanes l and l + 32 hold the
// two halves of one position's channels; one v_permlane32_swap per packed dword
// gives lane l channels 16 pr + 0..7 and lane l + 32 channels 16 pr + 8..15, so a
// store covers 32 contiguous bytes of each position instead of two 8-byte pieces.
template <int D>
__device__ __forceinline__ void store_dT_x16(uint16_t* dst_row, const f32x16& acc, float scale, int half) {
  static_assert(D == 16 || D == 32, "two channel groups per 16-channel pair");
#pragma unroll
  for (int pr = 0; pr < D / 16; ++pr) {
    const int g0 = 2 * pr, g1 = 2 * pr + 1;
    const uint32_t a0 = pack_bf16(acc[4 * g0] * scale, acc[4 * g0 + 1] * scale);
    const uint32_t a1 = pack_bf16(acc[4 * g0 + 2] * scale, acc[4 * g0 + 3] * scale);
    const uint32_t b0 = pack_bf16(acc[4 * g1] * scale, acc[4 * g1 + 1] * scale);
    const uint32_t b1 = pack_bf16(acc[4 * g1 + 2] * scale, acc[4 * g1 + 3] * scale);
    // lanes 0..31: {own, partner's} group g0; lanes 32..63: {partner's, own} group g1
    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    *reinterpret_cast<u32x4*>(dst_row + 16 * pr + 8 * half) = u32x4{s0[0], s1[0], s0[1], s1[1]};
  }
}

}  // namespace mfma
}  // namespace evo
