// Building blocks of the pipelined bf16 MFMA kernels (gfx950): direct
// global -> LDS copies, the swizzled LDS layout of staged [position][d] tiles,
// the workgroup -> XCD mapping and the tiled, pre-scaled fp32 bias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_common.h"

namespace evo {
namespace pipe {

using namespace mfma;

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Loads through LDS byte addresses (32-bit LDS pointers let the compiler fold
// constant offsets into the instruction).
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) { return *reinterpret_cast<lds_u32x4*>(addr); }
__device__ __forceinline__ u32x2 lds_load_tr(uint32_t addr) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4*>(addr)));
}
// The 16 accumulator registers of a 32-row tile read from an fp32 row vector in
// LDS: rows 8g + 4 half + (0..3).
__device__ __forceinline__ f32x16 lds_acc_rows(uint32_t addr, int half) {
  f32x16 c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<lds_f32x4*>(addr + 4 * (8 * g + 4 * half));
    c[4 * g + 0] = x[0];
    c[4 * g + 1] = x[1];
    c[4 * g + 2] = x[2];
    c[4 * g + 3] = x[3];
  }
  return c;
}

// Direct global -> LDS copies (global_load_lds_dword / _dwordx4): lane l's 4 or 16
// bytes land at lds_wave_base + 4 l or + 16 l (checked on gfx950 hardware).
// lds_wave_base is an LDS byte address, uniform across the wave.  The copies
// count in vmcnt like loads.  They are issued from inline assembly so that the
// compiler does not serialise every later LDS read behind them: the kernels
// order them explicitly with wait_vmcnt + barrier.  M0 is saved and restored.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_wave_base)
      : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_wave_base)
      : "memory");
}

// The same copies with a uniform 64-bit base (SGPRs) plus a per-lane 32-bit byte
// offset, which needs no per-lane address arithmetic.
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_wave_base)
      : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_wave_base)
      : "memory");
}

// A pointer that is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Makes the compiler wait here for the loads that produced x.  Registers loaded
// before a loop that also issues the (compiler-invisible) direct copies would
// otherwise be waited for inside the loop, with a count that also drains the
// copies in flight.
template <typename T>
__device__ __forceinline__ void retire(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the host pass cannot place 512-bit operands)
  asm volatile("" ::"v"(x));
#endif
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(p)));
}

// Waits until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroups are dispatched to the 8 XCDs round robin (block b runs on XCD b % 8),
// and each XCD has its own L2.  This maps the hardware block index to a logical
// index such that every XCD receives one contiguous range of logical blocks, so
// blocks that share data (same head, neighbouring rows) share an L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
  const int xcd = b & 7, slot = b >> 3;
  const int q = nblocks >> 3, rem = nblocks & 7;
  return xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
}

// ---------------------------------------------------------------- staged tiles
// A staged tile holds kBlk positions x D channels of bf16, row-major by
// position (2*D bytes per position), in 16-byte chunks.  Chunk p of position x
// is stored in slot p ^ swz(x) of that position's row so that the MFMA operand
// reads (16 consecutive positions, same chunk) and the transposing reads hit
// distinct LDS banks.
constexpr int kBlk = 64;  // positions per pipeline stage

template <int D, int POS = kBlk>
struct Tile {
  static constexpr int CHUNKS = D / 8;            // 16-byte chunks per position
  static constexpr int BYTES = POS * D * 2;       // bytes per staged tile of POS positions
  static constexpr int ROWS_PER_256B = 128 / D;   // positions per 256 bytes
  __device__ __forceinline__ static int swz(int x) {
    return CHUNKS > 1 ? (x / ROWS_PER_256B) & (CHUNKS - 1) : 0;
  }
  // Byte offset of chunk p of position x.
  __device__ __forceinline__ static int chunk_off(int x, int p) { return x * (2 * D) + ((p ^ swz(x)) << 4); }
  // Byte offset of channel c (multiple of 4) of position x: 8 bytes hold c..c+3.
  __device__ __forceinline__ static int quad_off(int x, int c) {
    return x * (2 * D) + (((c >> 3) ^ swz(x)) << 4) + ((c & 7) << 1);
  }
};

// Lane-dependent byte offsets of the MFMA operand reads of a staged tile,
// computed once per kernel.  Adding a multiple of 16 positions to a read keeps
// its swizzle, so every read of the main loop is one of these offsets plus a
// compile-time constant.
template <int D>
struct TileReads {
  static constexpr int KS = Shape<D>::KS, DB = Shape<D>::DB;
  int rows[KS];    // A operand (rows m = positions 0..31, k = channels 16 ks + 8 half ..)
  int tr[DB][2];   // transposing reads of positions 4 (lane / 32) + (lane % 16) / 4 (+ 8)
  __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      rows[ks] = Tile<D>::chunk_off(lane & 31, D < 16 ? 0 : 2 * ks + half);
    const int i = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      int c = db * 32 + (lane & 16) + 4 * (i & 3);
      if (c >= D) c &= (D - 1);  // channels >= D only feed result rows that are never used
      const int x = 4 * half + (i >> 2);
      tr[db][0] = Tile<D>::quad_off(x, c);
      tr[db][1] = Tile<D>::quad_off(x + 8, c);
    }
  }
  // A operand: rows = positions x0 + 0..31 (x0 a multiple of 16), k = channels of step ks.
  // `tile` is the LDS byte address of the staged tile.
  __device__ __forceinline__ u32x4 rows_operand(uint32_t tile, int x0, int ks, int lane) const {
    const u32x4 v = lds_load16(tile + rows[ks] + x0 * (2 * D));
    if (D < 16 && (lane >> 5)) return u32x4{0u, 0u, 0u, 0u};
    return v;
  }
  // At d = 8 the operand's k slots 8..15 (lanes 32..63) are free: the same read,
  // with `extra` in those lanes (for instance the split operands of the per-row
  // terms, so that they ride in the same MFMA).
  __device__ __forceinline__ u32x4 rows_operand_with(uint32_t tile, int x0, int lane, u32x4 extra) const {
    static_assert(D == 8, "k slots 8..15 are free only at d = 8");
    const u32x4 v = lds_load16(tile + rows[0] + x0 * (2 * D));
    return (lane >> 5) ? extra : v;
  }
  // A operand: rows = channels 32 db + (lane & 31), k = 16 positions p0 + 16 t + the
  // permutation of MFMA accumulator registers 8t..8t+7 (ds_read_b64_tr_b16), so
  // those registers of a tile whose rows are the positions p0.., packed to bf16,
  // are the matching B operand.
  __device__ __forceinline__ u32x4 tr_operand(uint32_t tile, int db, int p0, int t) const {
    const uint32_t base = tile + (p0 + 16 * t) * (2 * D);
    const u32x2 lo = lds_load_tr(base + tr[db][0]);
    const u32x2 hi = lds_load_tr(base + tr[db][1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// Direct copies of one pipeline stage: NT staged tiles, tile i holding positions
// x0 .. x0 + POS - 1 of the (row, head) slab that starts at byte pointer base[i].
// The stage's 16-byte chunks are spread over the workgroup's THREADS threads in
// LDS order.  Full blocks use the uniform-base form; the last, partial block reads
// positions >= n from position n - 1 (values that are never used with a nonzero
// weight).  Every wave issues exactly NIT copies per stage, so that waits can
// count them: a wave without chunks left issues a dummy copy into the 1 KB
// `dummy` LDS area (contents never read).
template <int D, int NT, int POS = kBlk, int THREADS = 256>
struct Stager {
  static constexpr int CH = Tile<D>::CHUNKS;
  static constexpr int PER_TILE = POS * CH;
  static constexpr int TOTAL = NT * PER_TILE;                  // chunks per stage
  static constexpr int NIT = (TOTAL + THREADS - 1) / THREADS;  // copies per thread per stage
  static_assert(TOTAL % 64 == 0, "stage must be a multiple of 64 chunks");
  uint32_t voff[NIT];  // byte offset of the chunk from position x0 of its slab
  uint32_t pstride;    // bytes between consecutive positions

  // Position and byte offset within the position of the chunk that copy `it` of
  // this lane writes.
  __device__ __forceinline__ static void chunk_of(int it, int wave, int lane, int& x, int& cbyte) {
    const int within = (it * THREADS + wave * 64 + lane) % PER_TILE;
    x = within / CH;
    cbyte = ((within % CH) ^ Tile<D>::swz(x)) * 16;
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
  // Tile index of copy `it` of `wave` (uniform; a compile-time constant when a
  // tile spans whole multiples of the workgroup's chunks).
  template <int IT>
  __device__ __forceinline__ static int tile_of(int wave) {
    if constexpr (PER_TILE % THREADS == 0) return IT * THREADS / PER_TILE;
    else return min((IT * THREADS + wave * 64) / PER_TILE, NT - 1);
  }
  template <int IT>
  __device__ __forceinline__ void issue_one(uint32_t lds, const char* const (&base)[NT], int x0, bool full,
                                            int n, int wave, uint32_t dummy) const {
    if (TOTAL % THREADS != 0 && IT * THREADS + wave * 64 >= TOTAL) {
      copy16_to_lds(uniform_ptr(base[0]), 0u, dummy);
      return;
    }
    const uint32_t dst = lds + (IT * THREADS + wave * 64) * 16;
    if constexpr (PER_TILE < 64) {
      // A wave's 64 chunks span several tiles: per-lane tile and address.
      const int lane = static_cast<int>(threadIdx.x & 63);
      const int ti = (IT * THREADS + wave * 64 + lane) / PER_TILE;
      const char* b = base[0];
#pragma unroll
      for (int i = 1; i < NT; ++i) b = ti == i ? base[i] : b;
      int x, cbyte;
      chunk_of(IT, wave, lane, x, cbyte);
      const int pos = full ? x0 + x : min(x0 + x, n - 1);
      copy16_to_lds(b + static_cast<size_t>(pos) * pstride + cbyte, dst);
      return;
    }
    // Only tiles LO..HI can hold copy IT of some wave: select among those (a
    // select over the whole array can end up as an indexed scratch access).
    constexpr int LO = IT * THREADS / PER_TILE;
    constexpr int HI = (IT * THREADS + THREADS - 64) / PER_TILE < NT - 1 ? (IT * THREADS + THREADS - 64) / PER_TILE
                                                                         : NT - 1;
    const int ti = tile_of<IT>(wave);
    const char* b = base[LO];
#pragma unroll
    for (int i = LO + 1; i <= HI; ++i)
      if (ti == i) b = base[i];
    if (full) {
      copy16_to_lds(uniform_ptr(b + static_cast<size_t>(x0) * pstride), voff[IT], dst);
    } else {
      int x, cbyte;
      chunk_of(IT, wave, static_cast<int>(threadIdx.x & 63), x, cbyte);
      const int pos = min(x0 + x, n - 1);
      copy16_to_lds(b + static_cast<size_t>(pos) * pstride + cbyte, dst);
    }
  }
  template <int IT = 0>
  __device__ __forceinline__ void issue(uint32_t lds, const char* const (&base)[NT], int x0, int n, int wave,
                                        uint32_t dummy = 0) const {
    if constexpr (IT < NIT) {
      issue_one<IT>(lds, base, x0, x0 + POS <= n, n, wave, dummy);
      issue<IT + 1>(lds, base, x0, n, wave, dummy);
    }
  }
};

// ---------------------------------------------------------------- tiled bias
// The pre-scaled bias sqrt(d) * bias[h][j][k] in fp32, stored as 32 x 32 tiles in
// the MFMA accumulator order, so that one accumulator tile is four fully
// coalesced 1 KB loads.  Orientation 0 ("query lanes"): accumulator rows are
// keys and lanes are queries (S^T tiles).  Orientation 1 ("key lanes"): rows are
// queries, lanes are keys (S tiles).  Tile (qt, kt) of head h starts at float
// ((h * nt + qt) * nt + kt) * 1024; inside it, register v = 4 g + e of lane l is
// float g * 256 + 4 l + e.  Keys >= N hold -inf, queries >= N hold 0.
__device__ __forceinline__ int64_t bias_tile_offset(int h, int qt, int kt, int nt) {
  return ((static_cast<int64_t>(h) * nt + qt) * nt + kt) * 1024;
}

// One 32 x 32 bias tile (query tile qt, key tile kt) of head h, by one 256-thread
// workgroup: the block is read once (coalesced rows of 32 keys) into LDS, then
// written in the query-lane order to out_q and in the key-lane order to out_k
// (each skipped when NULL), each as 256 coalesced 16-byte stores.
template <typename T>
__device__ __forceinline__ void bias_tile(const Problem& p, const T* __restrict__ bias, float* __restrict__ out_q,
                                          float* __restrict__ out_k, int nt, int tile) {
  __shared__ float tile_lds[32][33];  // [query][key], padded
  const int kt = tile % nt;
  const int qt = (tile / nt) % nt;
  const int h = tile / (nt * nt);
  const float sd = sqrtf(static_cast<float>(p.D));
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int jj = (t >> 5) + 8 * i, kk = t & 31;
    const int j = qt * 32 + jj, k = kt * 32 + kk;
    float val;
    if (k >= p.N) {
      val = -INFINITY;
    } else if (j >= p.N || bias == nullptr) {
      val = 0.f;
    } else {
      val = sd * Elem<T>::load(bias, (static_cast<int64_t>(h) * p.N + j) * p.N + k);
    }
    tile_lds[jj][kk] = val;
  }
  __syncthreads();
  // Thread t writes floats 4t..4t+3 of the tile: register group g = t / 64 of lane
  // l = t % 64, accumulator rows 8g + 4(l / 32) + e, column l % 32.
  const int g = t >> 6, lane = t & 63;
  const int row0 = 8 * g + 4 * (lane >> 5), col = lane & 31;
  const int64_t off = (((static_cast<int64_t>(h) * nt + qt) * nt + kt) * 1024) + 4 * t;
  if (out_q)  // query lanes: rows are keys, the column is the query
    *reinterpret_cast<float4*>(out_q + off) =
        make_float4(tile_lds[col][row0], tile_lds[col][row0 + 1], tile_lds[col][row0 + 2], tile_lds[col][row0 + 3]);
  if (out_k)  // key lanes: rows are queries, the column is the key
    *reinterpret_cast<float4*>(out_k + off) =
        make_float4(tile_lds[row0][col], tile_lds[row0 + 1][col], tile_lds[row0 + 2][col], tile_lds[row0 + 3][col]);
}

__device__ __forceinline__ f32x16 load_bias_tile(const float* __restrict__ tile, int lane) {
  // The tile address is the same in every lane: as a scalar base plus a 32-bit
  // lane offset the loads need no per-lane 64-bit address arithmetic.  The global
  // address space keeps them global (not flat) loads, which count in vmcnt only,
  // so waits for LDS reads do not also wait for them.
  typedef __attribute__((address_space(1))) const char gchar;
  typedef __attribute__((address_space(1))) const f32x4 gf32x4;
  gchar* base = (gchar*)(uniform_ptr(tile));
  const uint32_t off = static_cast<uint32_t>(lane) * 16;
  f32x16 c;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *reinterpret_cast<gf32x4*>(base + off + g * 1024);
    c[4 * g + 0] = x[0];
    c[4 * g + 1] = x[1];
    c[4 * g + 2] = x[2];
    c[4 * g + 3] = x[3];
  }
  return c;
}

}  // namespace pipe

// Number of 32-wide tiles per axis of the tiled bias (positions padded to 128).
inline int bias_tiles(int n) { return (n + 127) / 128 * 4; }
size_t tiled_bias_bytes(const Problem& p);
// Writes the tiled, sqrt(d)-scaled fp32 bias in the query-lane order to out_q and
// in the key-lane order to out_k (see above); either may be NULL.
hipError_t launch_bias_tiles(const Problem& p, const void* bias, float* out_q, float* out_k, hipStream_t s);
// Forward pre-pass: the tiled bias in the query-lane order and, if mask is not
// NULL, the per-key split mask operands kaug [R,N] x 16 B and the last live key
// of each row last_live [R] (kernels_bias_prep.hip).
hipError_t launch_fwd_prep(const Problem& p, const void* bias, const float* mask, float* out_q, void* kaug,
                           int* last_live, hipStream_t s);
// dQ, dK, dV in one pass (kernels_bwd_fused.hip), for head_dim <= 32 and N <= 384;
// needs the per-row split operands (qaug, kaug) and the key-lane bias tiles.
// Queries per attention row in the backward's pre-formed query operands (qops):
// N rounded up to 128, so that every 32-query block of a 128-query tile exists.
// Layout per (r, h): blocks of 32 queries, each 32 S-step operands
// [-a, -a, -a, 1, 1, 1, 0, 0] (a = sqrt(d) lse, split) then 32 dP-step operands
// [-D, -D, -D, 0, ...]; padding queries hold the dead-query S operand.
__host__ __device__ inline int qops_queries(int n) { return (n + 127) / 128 * 128; }

// Compute units of the current device (cached per device).
int device_cus();
// dbias[i] = sum over groups g = 0, 1, ... of part[g][i], in increasing g, for the
// elements i = first, first + stride, ... (in units of four elements when n is a
// multiple of 4, so that every group's partial stays 16-byte aligned).  All groups'
// loads of an element are issued before the first add (groups <= kMaxDbiasGroups).
constexpr int kMaxDbiasGroups = 16;
__device__ __forceinline__ void dbias_reduce_range(const float* __restrict__ part, int groups, int64_t n,
                                                   float* __restrict__ dbias, int64_t first, int64_t stride) {
  const int64_t n4 = n % 4 == 0 ? n / 4 : 0;
  for (int64_t i = first; i < n4; i += stride) {
    float4 v[kMaxDbiasGroups];
#pragma unroll
    for (int g = 0; g < kMaxDbiasGroups; ++g)
      if (g < groups) v[g] = reinterpret_cast<const float4*>(part + static_cast<int64_t>(g) * n)[i];
    float4 s = v[0];
#pragma unroll
    for (int g = 1; g < kMaxDbiasGroups; ++g)
      if (g < groups) {
        s.x += v[g].x;
        s.y += v[g].y;
        s.z += v[g].z;
        s.w += v[g].w;
      }
    reinterpret_cast<float4*>(dbias)[i] = s;
  }
  // (otherwise one element per thread)
  for (int64_t i = 4 * n4 + first; i < n; i += stride) {
    float s = part[i];
    for (int g = 1; g < groups; ++g) s += part[static_cast<int64_t>(g) * n + i];
    dbias[i] = s;
  }
}

bool bwd_fused_supported(const Problem& p);
// The fused dQ, dK, dV pass.  With dbias_part non-null it also forms a.dbias from
// the dbias_groups partial sums at dbias_part (the dBias pass runs before it) once
// its rows are done.
hipError_t launch_bwd_fused(const Problem& p, const BwdArgs& a, const float* bias_k, const float* dbias_part,
                            int dbias_groups, hipStream_t s);
// bf16 forward for head_dim 8, 16, 32 (kernels_fwd_pp.hip).
hipError_t launch_fwd_pp(const Problem& p, const FwdArgs& a, float* bias_t, void* kaug, int* last_live,
                         hipStream_t s);

}  // namespace evo

namespace evo {
namespace pipe {

// ---------------------------------------------------------------- per-row terms
// Per-row terms (the key mask, the logsumexp, the softmax Jacobian's D) enter the
// MFMA accumulators through one extra 16-deep step instead of vector ALU work:
// the query side and the key side each hold 8 bf16 values in the k slots 0..7
// (lanes 0..31; lanes 32..63 are the k slots 8..15), and their product is
//   sum_k q_aug[k] key_aug[k].
// The key side is zero in lanes 32..63, so the query side may hold anything
// finite there.  A finite float x is carried exactly as the sum of three bf16
// parts obtained by truncation: hi = top 16 bits of x, mid = top 16 bits of
// x - hi, lo = x - hi - mid (at most 8 significant bits, so exact in bf16).
struct Split3 {
  uint32_t hi, mid, lo;  // bf16 bit patterns in the low 16 bits
};
__device__ __forceinline__ Split3 split3(float x) {
  const uint32_t h = __float_as_uint(x) & 0xffff0000u;
  const float r1 = x - __uint_as_float(h);
  const uint32_t m = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(m);
  return Split3{h >> 16, m >> 16, __float_as_uint(r2) >> 16};
}

constexpr uint32_t kBf16One = 0x3f80u;
constexpr float kHuge = 1e30f;  // stands in for infinity in the split operands

// Key side of the logits: k slots [1, 1, 1, m, m, m, 0, 0] (m = sqrt(d) * mask,
// a masked key's -inf replaced by -1e30), zero in lanes 32..63.
__device__ __forceinline__ u32x4 key_aug(float m_scaled, int lane) {
  const Split3 m = split3(fmaxf(m_scaled, -kHuge));
  const u32x4 v = {kBf16One | (kBf16One << 16), kBf16One | (m.hi << 16), m.mid | (m.lo << 16), 0u};
  return (lane >> 5) ? u32x4{0u, 0u, 0u, 0u} : v;
}
// Key side of dP: [1, 1, 1, 0, 0, 0, 0, 0], zero in lanes 32..63.
__device__ __forceinline__ u32x4 key_aug_unit(int lane) {
  const u32x4 v = {kBf16One | (kBf16One << 16), kBf16One, 0u, 0u};
  return (lane >> 5) ? u32x4{0u, 0u, 0u, 0u} : v;
}
// Query side of the logits: [-a, -a, -a, 1, 1, 1, 0, 0] (a = sqrt(d) * lse, split).
// With key_aug this adds sqrt(d) * (mask - lse) to the logit accumulator.
__device__ __forceinline__ u32x4 query_aug_lse(float a) {
  const Split3 n = split3(-a);
  return u32x4{n.hi | (n.mid << 16), n.lo | (kBf16One << 16), kBf16One | (kBf16One << 16), 0u};
}
// Query side of dP: [-D, -D, -D, 0, 0, 0, 0, 0]; with key_aug_unit it adds -D.
__device__ __forceinline__ u32x4 query_aug_delta(float dlt) {
  const Split3 n = split3(-dlt);
  return u32x4{n.hi | (n.mid << 16), n.lo, 0u, 0u};
}

// sqrt(d) * lse as used by the query side: a query whose keys are all masked
// (lse = -inf), or a padding query, gets a huge finite value so that every
// probability of it is exactly 0 and no inf - inf arises.
__device__ __forceinline__ float lse_term(float lse, float sd, bool valid) {
  return (valid && lse != -INFINITY) ? sd * lse : kHuge;
}

// Query side of the logits for a padding query: -1e30 in the lse slots, so that
// its probabilities are exactly 0.
__device__ __forceinline__ u32x4 dead_query_aug() {
  const Split3 n = split3(-kHuge);
  return u32x4{n.hi | (n.mid << 16), n.lo | (kBf16One << 16), kBf16One | (kBf16One << 16), 0u};
}

// Direct copy of 64 consecutive 16-byte entries (one per lane) of a row vector
// starting at entry x0; entries past n read entry n - 1.
__device__ __forceinline__ void copy_rows16(const u32x4* row, int x0, int n, uint32_t dst, int lane) {
  if (x0 + 64 <= n)
    copy16_to_lds(uniform_ptr(row + x0), static_cast<uint32_t>(lane) * 16, dst);
  else
    copy16_to_lds(row + min(x0 + lane, n - 1), dst);
}

// Direct copy of 64 consecutive floats (one per lane) of a row vector starting at
// element x0; elements past n read element n - 1.
__device__ __forceinline__ void copy_row64(const float* row, int x0, int n, uint32_t dst, int lane) {
  if (x0 + 64 <= n)
    copy4_to_lds(uniform_ptr(row + x0), static_cast<uint32_t>(lane) * 4, dst);
  else
    copy4_to_lds(row + min(x0 + lane, n - 1), dst);
}

}  // namespace pipe
}  // namespace evo
