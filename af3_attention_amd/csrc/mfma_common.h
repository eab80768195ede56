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

// max(a, b, c) in one v_max3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// acc + lo(p) + hi(p) for a packed bf16 pair p, in one v_dot2_f32_bf16 with (1, 1).
__device__ __forceinline__ float add_bf16_pair(uint32_t p, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

// Maximum over the 32 values of two accumulator tiles, in four independent
// v_max3 chains.
__device__ __forceinline__ float tile_max(const f32x16& a, const f32x16& b) {
  float m[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m[u] = max3f(a[4 * u], a[4 * u + 1], a[4 * u + 2]);
    m[u] = max3f(m[u], a[4 * u + 3], b[4 * u]);
    m[u] = max3f(m[u], b[4 * u + 1], b[4 * u + 2]);
    m[u] = fmaxf(m[u], b[4 * u + 3]);
  }
  return max3f(m[0], m[1], fmaxf(m[2], m[3]));
}

// Workgroup barrier for LDS hand-off only: waits for this wave's LDS operations,
// not for its outstanding global loads (those are prefetches for a later step).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int64_t elem_offset(const Problem& p, int r, int pos, int h) {
  return ((static_cast<int64_t>(r) * p.row_stride + static_cast<int64_t>(pos) * p.pos_stride) * p.H + h) * p.D;
}

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kStep = 64;      // positions staged per pipeline step

template <int D>
struct Shape {
  static constexpr int KS = D >= 16 ? D / 16 : 1;  // 16-deep MFMA steps over d
  static constexpr int DB = D >= 32 ? D / 32 : 1;  // 32-row blocks over d for transposed outputs
  static constexpr int ROW = KS * 16 + 8;          // bf16 per staged [pos][d] row (8 padding)
  static constexpr int TRROW = KS * 16 + 16;       // row stride for arrays read with tr_operand
  static constexpr int TROW = kStep + 8;           // bf16 per staged [d][pos] row (8 padding)
  static constexpr int CHUNKS = D / 8;             // 16-byte chunks per position
  static constexpr int LOADS = (kStep * CHUNKS + kThreads - 1) / kThreads;  // chunks per thread
};

// kStep positions of one (row, head) of a [.., H, D] bf16 tensor, held in
// registers between the global load and the LDS store, so the load of the next
// step overlaps the compute of the current one.  Each thread owns fixed
// 16-byte chunks; the per-step address is a uniform base plus a fixed 32-bit
// per-lane offset.  Loads are unconditional (positions past the end are
// clamped to the last one) so that no branch separates a prefetch from its
// consumer; the store writes zeros for positions >= N.
template <int D>
struct Stage {
  using S = Shape<D>;
  u32x4 val[S::LOADS];
  uint32_t off[S::LOADS];  // element offset of the chunk at step position pr
  uint32_t pstride;        // elements between consecutive positions
  int pr[S::LOADS];        // position of the chunk within the step (>= kStep: idle)

  __device__ __forceinline__ void init(const Problem& p) {
    pstride = static_cast<uint32_t>(p.pos_stride * p.H * D);
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
      const int c = threadIdx.x + i * kThreads;
      pr[i] = c < kStep * S::CHUNKS ? c / S::CHUNKS : kStep;
      const int ch = c % S::CHUNKS;
      off[i] = static_cast<uint32_t>(ch * 8);
    }
  }

  // base: element (r, p0, h, 0) of the tensor (uniform across the workgroup).
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int p0, int n) {
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
      const int pos = min(pr[i] < kStep ? pr[i] : 0, n - 1 - p0);
      val[i] = *reinterpret_cast<const u32x4*>(base + pos * pstride + off[i]);
    }
  }

  // rows: [pos][d] with row stride `row`; trans: [d][pos] with row stride TROW.
  __device__ __forceinline__ void store(uint16_t* rows, uint16_t* trans, int row, int p0, int n) const {
#pragma unroll
    for (int i = 0; i < S::LOADS; ++i) {
      if (pr[i] >= kStep) continue;
      const int ch = (threadIdx.x + i * kThreads) % S::CHUNKS;
      const u32x4 v = p0 + pr[i] < n ? val[i] : u32x4{0u, 0u, 0u, 0u};
      if (rows) *reinterpret_cast<u32x4*>(&rows[pr[i] * row + ch * 8]) = v;
      if (trans) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          trans[(ch * 8 + 2 * e) * S::TROW + pr[i]] = static_cast<uint16_t>(v[e] & 0xffffu);
          trans[(ch * 8 + 2 * e + 1) * S::TROW + pr[i]] = static_cast<uint16_t>(v[e] >> 16);
        }
      }
    }
  }
};

// Element offset of (r, pos, h, 0), split as a uniform part for (r, h) and a
// position stride, so loops over positions advance a uniform pointer.
__device__ __forceinline__ int64_t row_head_offset(const Problem& p, int r, int h) {
  return (static_cast<int64_t>(r) * p.row_stride * p.H + h) * p.D;
}
__device__ __forceinline__ int64_t pos_step(const Problem& p) { return p.pos_stride * p.H * p.D; }

// A operand (rows = 32 positions from pos0, k = d) from a staged [pos][d] array.
template <int D>
__device__ __forceinline__ u32x4 rows_operand(const uint16_t* rows, int pos0, int ks, int col, int half) {
  if (D < 16 && half == 1) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(&rows[(pos0 + col) * Shape<D>::ROW + ks * 16 + 8 * half]);
}

// ds_read_b64_tr_b16 (gfx950), checked on hardware: within each group of 16
// lanes, lane i receives element v (v = 0..3) from the address supplied by lane
// 4v + i/4, offset by i % 4 elements.  So if lane s supplies
// &M[row0 + s/4][col0 + 4 (s % 4)] of a row-major bf16 matrix M, lane i gets
// M[row0 + v][col0 + i] for v = 0..3: a column slice, i.e. a transposed read.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* addr) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(addr));
  return __builtin_bit_cast(u32x2, x);
}

// A operand (rows = d of block db, k = 16 positions p0 + 16 t + permutation)
// from a staged row-major [pos][d] array with row stride `row` elements, read
// with transposing loads.  The permutation is the one of accumulator registers
// 8t..8t+7 (positions p0 + 16t + 8(i/4) + 4(lane/32) + i%4), so those registers,
// packed to bf16, are the matching B operand.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const uint16_t* rows, int row, int db, int p0, int t, int lane) {
  const int i = lane & 15;
  int dbase = db * 32 + (lane & 16);
  if (D < 32 && dbase >= D) dbase = 0;  // rows d >= D of the result are never used
  const int pos = p0 + 16 * t + 4 * (lane >> 5) + (i >> 2);
  const uint16_t* a0 = rows + pos * row + dbase + 4 * (i & 3);
  const u32x2 lo = lds_read_tr(a0);
  const u32x2 hi = lds_read_tr(a0 + 8 * row);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// A operand (rows = d of block db, k = 16 positions p0 + 16 t + permutation) from a
// staged [d][pos] array.  The permutation is the one of accumulator registers
// 8t..8t+7, so those registers (packed to bf16) are the matching B operand.
template <int D>
__device__ __forceinline__ u32x4 trans_operand(const uint16_t* trans, int db, int p0, int t, int col, int half) {
  const uint16_t* row = &trans[(db * 32 + col) * Shape<D>::TROW];
  const int b = p0 + 16 * t + 4 * half;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(row + b);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(row + b + 8);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// B operand straight from global memory: position pos (the lane's column),
// d = 16 ks + 8 half + i.  Zero outside the tensor.
template <int D>
__device__ __forceinline__ u32x4 global_operand(const Problem& p, const uint16_t* src, int r, int pos, int h, int ks,
                                                int half) {
  const int d0 = ks * 16 + 8 * half;
  if (pos >= p.N || d0 >= D) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(src + elem_offset(p, r, pos, h) + d0);
}

// The 16 accumulator registers of a 32-row tile read from a row vector: rows
// 8g + 4 half + (0..3).
__device__ __forceinline__ f32x16 load_acc_rows(const float* base, int half) {
  f32x16 c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(base + 8 * g + 4 * half);
    c[4 * g + 0] = x[0];
    c[4 * g + 1] = x[1];
    c[4 * g + 2] = x[2];
    c[4 * g + 3] = x[3];
  }
  return c;
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

}  // namespace mfma

// Bias pre-pass shared by the MFMA kernels: out[h][j][k] (or out[h][k][j] when
// transpose_out) = sqrt(d) * bias[h][j][k] in fp32 over an np x np padded square;
// keys k >= N hold -inf and padded queries hold 0.
int bias_pad(int n);
hipError_t launch_bias_prep(const Problem& p, const void* bias, float* out, int np, int transpose_out,
                            hipStream_t s);

}  // namespace evo
