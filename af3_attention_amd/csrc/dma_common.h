// Direct global -> LDS copies (gfx950) and LDS operand reads through pointers.
//
// The copies (global_load_lds_dwordx4) are issued from inline assembly, so the
// compiler does not track them: it neither waits for them before LDS reads nor
// counts them in vmcnt (its conservative handling of such copies would place
// vmcnt(0) waits inside the main loops).  Kernels order them explicitly with
// wait_vm (the s_waitcnt builtin, so the compiler knows what a wait retired)
// and a workgroup barrier.  M0 is saved and restored around each copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pipe_common.h"

namespace evo {
namespace dma {

using namespace mfma;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

template <typename T>
__device__ __forceinline__ lds_char* lds_ptr(T& obj) {
  return (lds_char*)(&obj);
}

typedef __attribute__((address_space(1))) const f32x4 glb_f32x4;
typedef __attribute__((address_space(1))) const char glb_char;

// The 16 accumulator registers of a pre-tiled 32 x 32 bias tile (pipe::bias_tile_offset's
// layout): four coalesced 1 KB global loads from a uniform base.
__device__ __forceinline__ f32x16 load_tile_acc(const float* tile, int lane) {
  glb_char* base = (glb_char*)(pipe::uniform_ptr(tile)) + lane * 16;
  f32x16 c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<glb_f32x4*>(base + g * 1024);
    c[4 * g + 0] = x[0];
    c[4 * g + 1] = x[1];
    c[4 * g + 2] = x[2];
    c[4 * g + 3] = x[3];
  }
  return c;
}

// 16-byte LDS load.
__device__ __forceinline__ u32x4 ld16(const lds_char* p) { return *reinterpret_cast<lds_cu32x4*>(p); }
// Transposing 8-byte LDS load (ds_read_b64_tr_b16).
__device__ __forceinline__ u32x2 ld_tr(const lds_char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p)));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); the unused counters are left at their maximum.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier after this wave's LDS reads have returned (no memory fence:
// the copies a barrier publishes are retired by an explicit wait_vm before it).
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
}

// One 16-byte copy per lane: lane l's bytes land at dst + 16 l.  `dst` must be
// the same in every lane.
__device__ __forceinline__ void copy16(const void* src, lds_char* dst) {
  pipe::copy16_to_lds(src, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
}
// The same with a uniform 64-bit base and a per-lane byte offset.
__device__ __forceinline__ void copy16(const void* sbase, uint32_t voff, lds_char* dst) {
  pipe::copy16_to_lds(sbase, voff, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
}

// Copies of NT staged tiles of POS positions x D channels (the swizzled layout
// of pipe::Tile) into consecutive LDS tiles starting at dst.  Tile i holds
// positions x0 .. x0 + POS - 1 of the (row, head) slab that starts at byte
// pointer base[i]; positions >= n read position n - 1 (values that never get a
// nonzero weight).  The stage's 16-byte chunks are spread over THREADS threads
// in LDS order, NIT copies per thread.
template <int D, int NT, int POS = pipe::kBlk, int THREADS = 256>
struct Stager {
  static constexpr int CH = pipe::Tile<D, POS>::CHUNKS;
  static constexpr int PER_TILE = POS * CH;
  static constexpr int TOTAL = NT * PER_TILE;
  static constexpr int NIT = TOTAL / THREADS;
  static_assert(TOTAL % THREADS == 0, "stage must be a whole number of copies per thread");
  static_assert(PER_TILE % 64 == 0, "a wave's copy must stay within one tile");
  uint32_t voff[NIT];  // byte offset of this lane's chunk from position x0 of the slab
  uint32_t pstride;    // bytes between consecutive positions

  // Position within the tile and byte offset within the position of the chunk
  // that copy `it` of this lane writes.
  __device__ __forceinline__ static void chunk_of(int it, int wave, int lane, int& x, int& cbyte) {
    const int within = (it * THREADS + wave * 64 + lane) % PER_TILE;
    x = within / CH;
    cbyte = ((within % CH) ^ pipe::Tile<D, POS>::swz(x)) * 16;
  }

  __device__ __forceinline__ void init(int wave, int lane, uint32_t pstride_bytes) {
    pstride = pstride_bytes;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      int x, cbyte;
      chunk_of(it, wave, lane, x, cbyte);
      voff[it] = static_cast<uint32_t>(x) * pstride_bytes + cbyte;
    }
  }
  // Slab of this wave's copy IT (uniform; a compile-time choice when a tile spans
  // a whole number of the workgroup's copies, else scalar selects).
  template <int IT>
  __device__ __forceinline__ static const char* slab(const char* const (&base)[NT], int wave) {
    if constexpr (PER_TILE % THREADS == 0) {
      return base[IT * THREADS / PER_TILE];
    } else {
      const int ti = (IT * THREADS + wave * 64) / PER_TILE;
      uint64_t b = reinterpret_cast<uint64_t>(base[0]);
#pragma unroll
      for (int i = 1; i < NT; ++i) {
        const uint64_t bi = reinterpret_cast<uint64_t>(base[i]);
        b = ti == i ? bi : b;
      }
      return reinterpret_cast<const char*>(b);
    }
  }
  template <int IT = 0>
  __device__ __forceinline__ void issue_full(lds_char* dst, const char* const (&base)[NT], int x0, int wave) const {
    if constexpr (IT < NIT) {
      copy16(pipe::uniform_ptr(slab<IT>(base, wave) + static_cast<size_t>(x0) * pstride), voff[IT],
             dst + (IT * THREADS + wave * 64) * 16);
      issue_full<IT + 1>(dst, base, x0, wave);
    }
  }
  template <int IT = 0>
  __device__ __forceinline__ void issue_partial(lds_char* dst, const char* const (&base)[NT], int x0, int n,
                                                int wave) const {
    if constexpr (IT < NIT) {
      int x, cbyte;
      chunk_of(IT, wave, static_cast<int>(threadIdx.x & 63), x, cbyte);
      const int pos = min(x0 + x, n - 1);
      copy16(slab<IT>(base, wave) + static_cast<size_t>(pos) * pstride + cbyte, dst + (IT * THREADS + wave * 64) * 16);
      issue_partial<IT + 1>(dst, base, x0, n, wave);
    }
  }
  // Copies of the positions x0 .. x0 + POS - 1 of the slabs base[0..NT-1].
  __device__ __forceinline__ void issue(lds_char* dst, const char* const (&base)[NT], int x0, int n, int wave) const {
    if (x0 + POS <= n)
      issue_full(dst, base, x0, wave);
    else
      issue_partial(dst, base, x0, n, wave);
  }
};

// Lane-dependent byte offsets of the MFMA operand reads of a staged tile (the
// layout of pipe::Tile), computed once per kernel; the reads take an LDS pointer
// to the tile, so the compiler knows which stage object they read.
template <int D>
struct Reads {
  static constexpr int KS = Shape<D>::KS, DB = Shape<D>::DB;
  int rows[KS];
  int tr[DB][2];
  __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      rows[ks] = pipe::Tile<D>::chunk_off(lane & 31, D < 16 ? 0 : 2 * ks + half);
    const int i = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      int c = db * 32 + (lane & 16) + 4 * (i & 3);
      if (c >= D) c &= (D - 1);  // channels >= D only feed result rows that are never used
      const int x = 4 * half + (i >> 2);
      tr[db][0] = pipe::Tile<D>::quad_off(x, c);
      tr[db][1] = pipe::Tile<D>::quad_off(x + 8, c);
    }
  }
  // A operand: rows = positions x0 + 0..31 (x0 a multiple of 16), k = channels of step ks.
  __device__ __forceinline__ u32x4 rows_operand(const lds_char* tile, int x0, int ks, int lane) const {
    const u32x4 v = ld16(tile + rows[ks] + x0 * (2 * D));
    if (D < 16 && (lane >> 5)) return u32x4{0u, 0u, 0u, 0u};
    return v;
  }
  // A operand: rows = channels 32 db + (lane & 31), k = positions p0 + 16 t + the
  // permutation of accumulator registers 8t..8t+7 (see pipe::TileReads).
  __device__ __forceinline__ u32x4 tr_operand(const lds_char* tile, int db, int p0, int t) const {
    const lds_char* base = tile + (p0 + 16 * t) * (2 * D);
    const u32x2 lo = ld_tr(base + tr[db][0]);
    const u32x2 hi = ld_tr(base + tr[db][1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

}  // namespace dma
}  // namespace evo
