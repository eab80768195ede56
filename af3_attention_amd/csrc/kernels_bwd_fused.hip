// dQ, dK and dV of pair-biased 3D attention in one pass (bf16 MFMA, gfx950),
// for head_dim <= 32 and up to 384 keys per row.
//
// The backward recomputes the probabilities from the saved logsumexp instead of
// storing them (the pages' memory-efficient kernel runs in the forward and the
// backward: gist.science MegaFold technical summary, Methodik section 1
// "EvoFlash-3D").  With dS = P * (dP - D):
//   dV[k] = sum_j P[j,k] dO[j],  dK[k] = sum_j dS[j,k] Q[j] / sqrt(d),
//   dQ[j] = sum_k dS[j,k] K[k] / sqrt(d).
// Here every score tile's P, dP and dS are computed once and feed all three.
//
// The unit of work is one attention row r of one head h with all its keys, so
// every sum above completes inside one workgroup and nothing is accumulated
// across workgroups.  The grid is persistent: one workgroup per compute unit
// walks through its rows one after another.  The next row's K and V are copied
// into a second buffer in pieces over the current row's first blocks, and its
// first query block and mask values during the current row, so a workgroup never
// waits for a row to start; each workgroup starts its rows at a different query
// block, so that the row changes of different compute units fall at different
// times.
//  * 8 waves, two per SIMD.  The 12 key tiles of 32 keys are split so that each
//    SIMD carries three: wave w < 4 owns tiles w and w + 4, wave w >= 4 owns tile
//    w + 4 and also forms dQ (below).  Each wave keeps its tiles' dK, dV in
//    registers while the workgroup walks the row's queries in blocks of 32, and
//    stores them at the start of the next row (through LDS, as whole key rows).
//    Q, dO and the per-query operands of each block are staged by direct copies,
//    double buffered;
//  * tiles are S = Q K^T (queries x keys), so a lane holds one key:
//      S  = Q K^T + sqrt(d) bias + sqrt(d) (mask - lse)   (bias: accumulator input,
//           a tiled fp32 copy loaded one block ahead, S accumulating in place in
//           its registers; mask and lse: one extra MFMA step on split-bf16
//           operands, at d = 8 folded into the free k slots of the main step)
//      dP = dO V^T - D                                   (D: likewise)
//      P = exp2(S log2(e)/sqrt(d)),  dS = P dP
//    P and dS, packed to bf16 in registers, are the B operands of dV^T += dO^T P
//    and dK^T += Q^T dS (A operands: transposing LDS reads of dO and Q);
//  * each tile's dS goes to LDS as [key][query].  During the next block wave
//    w >= 4 forms quadrant w - 4 (16 channels x 16 queries) of dQ^T of the
//    finished query tile over all key tiles with v_mfma_f32_16x16x32_bf16, one
//    instruction per 32-key tile (A = K^T, read from LDS once per row and kept in
//    registers; B = dS^T from transposing LDS reads), and stores it.  The dS
//    tiles are double buffered, so one barrier per block orders everything;
//  * when the dBias pass has run first (it writes one partial sum per row group),
//    the workgroups add those partials up once their rows are done.

#include <algorithm>
#include <type_traits>
#include <utility>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kFw = 8;                // waves per workgroup
constexpr int kFThreads = 64 * kFw;
constexpr int kFTiles = 12;           // key tiles per row this kernel handles
constexpr int kFMaxKeys = 32 * kFTiles;
constexpr int kFq = 32;               // queries per block
constexpr int kDsBytes = 32 * 64;     // one dS tile: 32 keys x 32 queries, bf16

typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// f(integral_constant<int, I>) for I = I0 .. N - 1.
template <int I0, int N, typename F>
__device__ __forceinline__ void for_each_const(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>());
    for_each_const<I0 + 1, N>(f);
  }
}

__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Per key tile of a wave: the key-side split operand, the next row's mask value
// of the lane's key, the dK^T and dV^T accumulators and the bias of the current
// and the next block.
struct KeyTile {
  int kt;       // key tile index
  bool valid;   // kt < number of key tiles of the row
  u32x4 s_key;
  float mask_next;
  f32x16 dk, dv;
  f32x16 bias[2];
};

template <int D>
__global__ __launch_bounds__(kFThreads, 1) void bwd_fused_kernel(Problem p, BwdArgs a,
                                                                  const float* __restrict__ bias_k, int nt,
                                                                  const float* __restrict__ dbias_part,
                                                                  int dbias_groups) {
  constexpr int KS = Shape<D>::KS;
  static_assert(Shape<D>::DB == 1, "head_dim <= 32");
  constexpr int TQ = Tile<D, kFq>::BYTES;   // one staged tile of 32 queries
  constexpr int STAGE = 2 * TQ + 1024;      // Q, dO, the 32 queries' S-step and dP-step operands
  constexpr int KRES = kFMaxKeys * 2 * D;   // K (or V) of one row
  using StQ = Stager<D, 2, kFq, kFThreads>;
  using StK = Stager<D, 2, kFMaxKeys, kFThreads>;
  __shared__ __align__(16) char lds[2 * STAGE + (2 * kFTiles + 1) * kDsBytes + 4 * KRES + 1024];
  // The per-block buffers come first, so that their reads take the offsets of
  // the unrolled loops as immediates (a ds_read offset is below 64 KB).
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t stage0 = lds0;
  const uint32_t ds0 = stage0 + 2 * STAGE;
  const uint32_t ds_trash = ds0 + 2 * kFTiles * kDsBytes;  // dS of tiles past the row's keys
  const uint32_t kv0 = ds_trash + kDsBytes;                // K, V of a row; two buffers of 2 KRES
  const uint32_t dummy = kv0 + 4 * KRES;

  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int nkt = (p.N + 31) / 32;  // key tiles = query blocks
  const int np = qops_queries(p.N);
  const bool pair_wave = wave < 4;  // two key tiles; otherwise one tile and dQ
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t pstride = static_cast<uint32_t>(p.pos_stride * p.H * D * 2);

  // Rows of this workgroup: blockIdx.x, blockIdx.x + gridDim.x, ...; the rows
  // of one head are contiguous per XCD (its L2 then holds that head's bias).
  const int items = p.R * p.H;
  const int n_local = (items - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                      static_cast<int>(gridDim.x);
  struct Row {
    int r, h;
    int64_t rh;  // element offset of (r, position 0, h)
  };
  auto row_of = [&](int li) __attribute__((always_inline)) {
    const int logical = xcd_logical_block(static_cast<int>(blockIdx.x) + li * static_cast<int>(gridDim.x), items);
    Row w;
    w.h = logical / p.R;
    w.r = logical % p.R;
    w.rh = row_head_offset(p, w.r, w.h);
    return w;
  };

  TileReads<D> rd;
  rd.init(lane);

  const uint16_t* const qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* const dop = static_cast<const uint16_t*>(a.dout);
  const uint16_t* const kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* const vp = static_cast<const uint16_t*>(a.v);
  // Key side of the D step (at d = 8 in every lane: it rides in k slots 8..15).
  const u32x4 dp_key = D == 8 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u} : key_aug_unit(lane);

  // Tile A: w (w < 4) or w + 4; tile B: w + 4 (w < 4 only).  Invalid tiles (past
  // the row's keys) run on clamped, finite data and are never stored.
  KeyTile ta, tb;
  ta.kt = pair_wave ? wave : wave + 4;
  tb.kt = wave + 4;
  ta.valid = ta.kt < nkt;
  tb.valid = pair_wave && tb.kt < nkt;
  // The mask value of the lane's key in row r, loaded ahead; when the row starts
  // it becomes the key-side split operand [1, 1, 1, m, m, m, 0, 0] (m = sqrt(d)
  // mask split in three; zeros in lanes 32..63, except at d = 8 where the operand
  // rides in the k slots 8..15 of the product's own MFMA step).
  auto load_key_side = [&](KeyTile& t, int r) __attribute__((always_inline)) {
    const int key = min(t.kt * 32 + (lane & 31), p.N - 1);
    t.mask_next = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
  };
  auto start_tile = [&](KeyTile& t) __attribute__((always_inline)) {
    retire(t.mask_next);
    const Split3 sm = split3(fmaxf(sd * t.mask_next, -kHuge));
    const u32x4 op = {kBf16One | (kBf16One << 16), kBf16One | (sm.hi << 16), sm.mid | (sm.lo << 16), 0u};
    t.s_key = (half && D != 8) ? u32x4{0u, 0u, 0u, 0u} : op;
#pragma unroll
    for (int e = 0; e < 16; ++e) t.dk[e] = t.dv[e] = 0.f;
  };

  // Copies of query block b of row w (Q, dO, and the query-side operands by the
  // last wave).  The per-lane copy offsets are recomputed here rather than kept
  // live across the loop (the empty asm keeps the compiler from hoisting them).
  auto issue_block = [&](const Row& w, int b, uint32_t st) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const char* const base[2] = {uniform_ptr(reinterpret_cast<const char*>(qp + w.rh)),
                                 uniform_ptr(reinterpret_cast<const char*>(dop + w.rh))};
    StQ stq;
    stq.init(wave, l, pstride);
    stq.issue(st, base, b * kFq, p.N, wave, dummy);
    if (wave == kFw - 1) {
      const u32x4* qo = static_cast<const u32x4*>(a.qops) + 2 * (static_cast<int64_t>(w.r) * p.H + w.h) * np;
      copy16_to_lds(uniform_ptr(qo + b * 64), static_cast<uint32_t>(l) * 16, st + 2 * TQ);
    }
  };
  // Copies of row w's K and V into the buffer at kvb.
  auto issue_kv = [&](const Row& w, uint32_t kvb) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const char* const base[2] = {uniform_ptr(reinterpret_cast<const char*>(kp + w.rh)),
                                 uniform_ptr(reinterpret_cast<const char*>(vp + w.rh))};
    StK stk;
    stk.init(wave, l, pstride);
    stk.issue(kvb, base, 0, p.N, wave, dummy);
  };
  // The share of those copies issued at position j of the current row: copy IT
  // of every lane at position IT + 1 (all remaining ones at the last position).
  auto issue_kv_part = [&](const Row& w, uint32_t kvb, int jj, int n_pos) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const char* const base[2] = {uniform_ptr(reinterpret_cast<const char*>(kp + w.rh)),
                                 uniform_ptr(reinterpret_cast<const char*>(vp + w.rh))};
    StK stk;
    stk.init(wave, l, pstride);
    const bool full = kFMaxKeys <= p.N;
    for_each_const<0, StK::NIT>([&](auto it_c) __attribute__((always_inline)) {
      constexpr int IT = decltype(it_c)::value;
      if (jj == min(IT + 1, n_pos - 1)) stk.template issue_one<IT>(kvb, base, 0, full, p.N, wave, dummy);
    });
  };
  // sqrt(d) * bias of tile t's keys for the 32 queries of block b of head h.
  auto load_bias = [&](const KeyTile& t, f32x16& dst, int h, int b) __attribute__((always_inline)) {
    dst = load_bias_tile(bias_k + bias_tile_offset(h, b, min(t.kt, nt - 1), nt), lane);
  };

  // dQ: wave w >= 4 forms quadrant qd = w - 4 of dQ^T (channels d0 = 16 (qd & 1),
  // queries q0 = 16 (qd >> 1)); quadrants with d0 >= D hold nothing.
  const int qd = wave & 3;
  const int dq_d0 = 16 * (qd & 1), dq_q0 = 16 * (qd >> 1);
  const bool dq_wave = !pair_wave && dq_d0 < D;
  const int g4 = lane >> 4, i16 = lane & 15;
  int ca = dq_d0 + 4 * (i16 & 3);
  if (ca >= D) ca &= (D - 1);  // channels >= D only feed rows that are never stored
  const int offA0 = Tile<D>::quad_off(8 * g4 + (i16 >> 2), ca);
  const int offA1 = Tile<D>::quad_off(8 * g4 + 4 + (i16 >> 2), ca);
  const int offB0 = Tile<32>::quad_off(8 * g4 + (i16 >> 2), dq_q0 + 4 * (i16 & 3));
  const int offB1 = Tile<32>::quad_off(8 * g4 + 4 + (i16 >> 2), dq_q0 + 4 * (i16 & 3));
  // The A operands (K^T, this quadrant's channels) of all key tiles of a row,
  // read once its K is resident and kept in registers.
  u32x4 kT[kFTiles];
  auto load_kT = [&](uint32_t kres) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < kFTiles; ++kt) {
      const uint32_t ka = kres + kt * (32 * 2 * D);
      const u32x2 a0 = lds_load_tr(ka + offA0), a1 = lds_load_tr(ka + offA1);
      kT[kt] = u32x4{a0[0], a0[1], a1[0], a1[1]};
    }
  };
  // The quadrant for query block qb of row w, whose dS tiles are in buffer dsbuf:
  // a sum over all key tile slots (the slots past the row's keys hold zeros),
  // every read issued before the first product.
  auto dq_tile = [&](const Row& w, int qb, uint32_t dsbuf) __attribute__((always_inline)) {
    u32x4 dsT[kFTiles];
#pragma unroll
    for (int kt = 0; kt < kFTiles; ++kt) {
      const uint32_t da = dsbuf + kt * kDsBytes;
      const u32x2 b0 = lds_load_tr(da + offB0), b1 = lds_load_tr(da + offB1);
      dsT[kt] = u32x4{b0[0], b0[1], b1[0], b1[1]};
    }
    __builtin_amdgcn_sched_barrier(0);  // keep all reads ahead of the products
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kFTiles; ++kt) acc = mma16(kT[kt], dsT[kt], acc);
    // lane: query q0 + (lane & 15), channels d0 + 4 (lane >> 4) + 0..3
    const int q = qb * kFq + dq_q0 + i16;
    const int d = dq_d0 + 4 * g4;
    if (q < p.N && d < D) {
      const float sc = 1.f / sd;
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dq) + elem_offset(p, w.r, q, w.h) + d) =
          u32x2{pack_bf16(acc[0] * sc, acc[1] * sc), pack_bf16(acc[2] * sc, acc[3] * sc)};
    }
  };

  // Score tile (block b, key tile t), in three phases: (1) S and dP on the matrix
  // cores, (2) P and dS on the vector ALU, (3) dV, dK on the matrix cores and dS
  // into the dS buffer.
  struct Probs {
    u32x4 p[2], ds[2];
  };
  // (1) S accumulates in place in the bias registers (they hold this block's bias
  // tile and are free again once P is formed); the query-side operands are loaded
  // complete from the stage.  kres: the row's K (V follows at kres + KRES).
  auto phase1 = [&](uint32_t st, const KeyTile& t, f32x16& sacc, uint32_t kres) __attribute__((always_inline)) {
    const uint32_t tq = st, tdo = st + TQ;
    const int jl = lane & 31;
    const u32x4 s_q = lds_load16(st + 2 * TQ + jl * 16);
    const u32x4 dp_q = lds_load16(st + 2 * TQ + 512 + jl * 16);
    const uint32_t kt_lds = kres + t.kt * (32 * 2 * D), vt_lds = kt_lds + KRES;
    if constexpr (D == 8) {
      // The per-row terms ride in k slots 8..15 of the one MFMA step.
      sacc = mma(rd.rows_operand_with(tq, 0, lane, s_q), rd.rows_operand_with(kt_lds, 0, lane, t.s_key), sacc);
      return mma(rd.rows_operand_with(tdo, 0, lane, dp_q), rd.rows_operand_with(vt_lds, 0, lane, dp_key),
                 f32x16{});
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sacc = mma(rd.rows_operand(tq, 0, ks, lane), rd.rows_operand(kt_lds, 0, ks, lane), sacc);
    sacc = mma(s_q, t.s_key, sacc);
    f32x16 dp = mma(rd.rows_operand(tdo, 0, 0, lane), rd.rows_operand(vt_lds, 0, 0, lane), f32x16{});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      dp = mma(rd.rows_operand(tdo, 0, ks, lane), rd.rows_operand(vt_lds, 0, ks, lane), dp);
    dp = mma(dp_q, dp_key, dp);
    return dp;
  };
  auto phase2 = [&](const f32x16& sacc, const f32x16& dp) __attribute__((always_inline)) {
    Probs o;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(sacc[8 * u + e] * c1);
        dsv[e] = pv[e] * dp[8 * u + e];
      }
      o.p[u] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                     pack_bf16(pv[6], pv[7])};
      o.ds[u] = u32x4{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                      pack_bf16(dsv[6], dsv[7])};
    }
    return o;
  };
  auto phase3 = [&](uint32_t st, KeyTile& t, const Probs& pr, uint32_t dsbuf) __attribute__((always_inline)) {
    const uint32_t tq = st, tdo = st + TQ;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      t.dv = mma(rd.tr_operand(tdo, 0, 0, u), pr.p[u], t.dv);
      t.dk = mma(rd.tr_operand(tq, 0, 0, u), pr.ds[u], t.dk);
    }
    // dS to LDS as [key][query]: registers 8u .. 8u + 3 hold queries 16 u + 4 half
    // + 0..3, registers 8u + 4 .. 8u + 7 hold queries 16 u + 8 + 4 half + 0..3.
    const uint32_t dsw = t.valid ? dsbuf + t.kt * kDsBytes : ds_trash;
    const int x = lane & 31;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 4 * half)) =
          u32x2{pr.ds[u][0], pr.ds[u][1]};
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 8 + 4 * half)) =
          u32x2{pr.ds[u][2], pr.ds[u][3]};
    }
  };
  auto tile_row = [&](uint32_t st, KeyTile& t, f32x16& bias, uint32_t dsbuf, uint32_t kres)
                      __attribute__((always_inline)) {
    const f32x16 dp = phase1(st, t, bias, kres);
    phase3(st, t, phase2(bias, dp), dsbuf);
  };
  // The same through LDS (the 2 * 64 * D bytes at reg, free for this wave): the
  // tile is written as [key][channel] bf16 and read back so that each lane
  // stores 16 contiguous bytes and a store covers whole 2 * D-byte key rows
  // (instead of 8-byte pieces of 32 rows).  The 16-byte chunks of key row x sit
  // in the staged-tile swizzle (chunk c at slot c ^ swz(x)), so the 8-byte writes
  // of the 32 keys spread over the banks.
  auto store_tile_lds = [&](const Row& w, const KeyTile& t, uint32_t reg) __attribute__((always_inline)) {
    if (!t.valid) return;
    const int x = lane & 31;
    const f32x16* accs[2] = {&t.dv, &t.dk};
    const float scales[2] = {1.f, 1.f / sd};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (8 * g < D) {
          const f32x16& acc = *accs[m];
          *reinterpret_cast<lds_u32x2*>(reg + m * 64 * D + x * 2 * D + ((g ^ Tile<D>::swz(x)) * 16) + 8 * half) =
              u32x2{pack_bf16(acc[4 * g] * scales[m], acc[4 * g + 1] * scales[m]),
                    pack_bf16(acc[4 * g + 2] * scales[m], acc[4 * g + 3] * scales[m])};
        }
      }
    }
    uint16_t* const dst[2] = {static_cast<uint16_t*>(a.dv), static_cast<uint16_t*>(a.dk)};
    int l = lane;
    asm volatile("" : "+v"(l));  // (per-lane offsets recomputed here, not kept live across rows)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int part = 0; part * 1024 < 64 * D; ++part) {
        const int byte = part * 1024 + l * 16;
        const int kx = byte / (2 * D), c = byte % (2 * D) / 16;  // key row and 16-byte chunk
        const int key = t.kt * 32 + kx, ch = 8 * c;
        const u32x4 v = lds_load16(reg + m * 64 * D + kx * 2 * D + ((c ^ Tile<D>::swz(kx)) * 16));
        if (byte < 64 * D && key < p.N)
          *reinterpret_cast<u32x4*>(dst[m] + elem_offset(p, w.r, key, w.h) + ch) = v;
      }
    }
  };
  auto store_tile = [&](const Row& w, const KeyTile& t) __attribute__((always_inline)) {
    const int key = t.kt * 32 + (lane & 31);
    if (!t.valid || key >= p.N) return;
    const int64_t off = elem_offset(p, w.r, key, w.h);
    store_dT<D>(static_cast<uint16_t*>(a.dv) + off, &t.dv, 1.f, half);
    store_dT<D>(static_cast<uint16_t*>(a.dk) + off, &t.dk, 1.f / sd, half);
  };

  // The blocks of all rows of this workgroup form one sequence g = 0, 1, ...
  // (position j of local row li); stage and dS buffers alternate with g, the K/V
  // buffer with li.  A workgroup visits the query blocks of every row starting at
  // block b0 = blockIdx.x mod nkt (the order of the sums over blocks is fixed per
  // workgroup), so that the row changes, with their bursts of K, V loads and
  // dK, dV stores, are spread over time across the compute units.  Step g:
  // everything issued one step earlier has arrived and every wave has finished
  // step g - 1 (its stage and dS tiles are complete; the buffers of step g - 2
  // are free).  Step g + 1's copies and bias start at once; the next row's K, V
  // copies are issued piecewise over the first steps of the current row, into
  // the buffer of the row before.  The two roles run separate copies of the loop
  // (the same number of barriers), so that neither role's registers have to be
  // reconciled with the other's.
  const int total = n_local * nkt;
  const int b0 = static_cast<int>(blockIdx.x) % nkt;
  auto blk = [&](int j) __attribute__((always_inline)) {
    const int x = j + b0;
    return x >= nkt ? x - nkt : x;
  };
  Row cur = row_of(0), prev = cur, nxt = cur;
  int j = 0, li = 0;
  auto step = [&](int g, auto s_c, auto pair_c) __attribute__((always_inline)) {
    constexpr int s = decltype(s_c)::value;
    constexpr bool PAIR = decltype(pair_c)::value;
    wait_vmcnt<0>();
    barrier();
    retire(ta.bias[s]);
    if constexpr (PAIR) retire(tb.bias[s]);
    const uint32_t kres = kv0 + (li & 1) * (2 * KRES);
    const bool more_rows = li + 1 < n_local;
    if (j == 0) {
      if (li > 0) {
        // The previous row's dK, dV are complete: store them (through the K/V
        // buffer of the row before, which is free until the next copies into
        // it), take this row's key-side operands.
        const uint32_t reg = kv0 + ((li + 1) & 1) * (2 * KRES) + (PAIR ? wave * 256 * D : 1024 * D + (wave - 4) * 128 * D);
        if (nkt >= 2) {
          store_tile_lds(prev, ta, reg);
          if constexpr (PAIR) store_tile_lds(prev, tb, reg + 128 * D);
        } else {
          store_tile(prev, ta);
          if constexpr (PAIR) store_tile(prev, tb);
        }
        start_tile(ta);
        if constexpr (PAIR) start_tile(tb);
      }
      if (more_rows) nxt = row_of(li + 1);
    }
    if (g + 1 < total) {
      const bool row_end = j + 1 == nkt;
      const Row& nr = row_end ? nxt : cur;
      const int nb = blk(row_end ? 0 : j + 1);
      issue_block(nr, nb, stage0 + (s ^ 1) * STAGE);
    }
    if (more_rows) {
      issue_kv_part(nxt, kv0 + ((li + 1) & 1) * (2 * KRES), j, nkt);
      if (j == min(1, nkt - 1)) {
        load_key_side(ta, nxt.r);
        if constexpr (PAIR) load_key_side(tb, nxt.r);
      }
    }
    const uint32_t st = stage0 + s * STAGE, dsb = ds0 + s * (kFTiles * kDsBytes);
    auto late_bias = [&]() __attribute__((always_inline)) {
      if (g + 1 < total) {
        const bool row_end = j + 1 == nkt;
        const Row& nr = row_end ? nxt : cur;
        const int nb = blk(row_end ? 0 : j + 1);
        __builtin_amdgcn_sched_barrier(0);
        load_bias(ta, ta.bias[s ^ 1], nr.h, nb);
        if constexpr (PAIR) load_bias(tb, tb.bias[s ^ 1], nr.h, nb);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (PAIR) {
      tile_row(st, ta, ta.bias[s], dsb, kres);
      late_bias();
      tile_row(st, tb, tb.bias[s], dsb, kres);
    } else {
      if (dq_wave) {
        if (g >= 1) {
          const uint32_t dsp = ds0 + (s ^ 1) * (kFTiles * kDsBytes);
          if (j == 0)
            dq_tile(prev, blk(nkt - 1), dsp);
          else
            dq_tile(cur, blk(j - 1), dsp);
        }
        if (j == 0) load_kT(kres);
      }
      late_bias();
      tile_row(st, ta, ta.bias[s], dsb, kres);
    }
  };
  auto advance = [&]() __attribute__((always_inline)) {
    if (++j == nkt) {
      j = 0;
      ++li;
      prev = cur;
      cur = nxt;
    }
  };
  auto run = [&](auto pair_c) __attribute__((always_inline)) {
    constexpr bool PAIR = decltype(pair_c)::value;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    load_bias(ta, ta.bias[0], cur.h, blk(0));
    if constexpr (PAIR) load_bias(tb, tb.bias[0], cur.h, blk(0));
    for (int g = 0; g < total; g += 2) {
      step(g, I0(), pair_c);
      advance();
      if (g + 1 < total) {
        step(g + 1, I1(), pair_c);
        advance();
      }
    }
    wait_vmcnt<0>();
    barrier();
    // (prev is now the last row)
    if constexpr (!PAIR) {
      if (dq_wave) dq_tile(prev, blk(nkt - 1), ds0 + ((total - 1) & 1) * (kFTiles * kDsBytes));
    }
    const uint32_t reg = kv0 + (n_local & 1) * (2 * KRES) + (PAIR ? wave * 256 * D : 1024 * D + (wave - 4) * 128 * D);
    store_tile_lds(prev, ta, reg);
    if constexpr (PAIR) store_tile_lds(prev, tb, reg + 128 * D);
  };

  // Prologue: the first row's key-side operands, its K and V, its first query
  // block.
  load_key_side(ta, cur.r);
  if (pair_wave) load_key_side(tb, cur.r);
  start_tile(ta);
  if (pair_wave) start_tile(tb);
  // dS slots of tiles past the row's keys are zero in both buffers (no tile
  // writes them), so that the dQ sums may run over all slots.
  for (int i = threadIdx.x; i < 2 * (kFTiles - nkt) * (kDsBytes / 16); i += kFThreads) {
    const int slot = nkt + i / (kDsBytes / 16) % (kFTiles - nkt), buf = i / ((kFTiles - nkt) * (kDsBytes / 16));
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(ds0 + buf * (kFTiles * kDsBytes) + slot * kDsBytes +
                                                                 (i % (kDsBytes / 16)) * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  issue_kv(cur, kv0);
  issue_block(cur, blk(0), stage0);
  if (pair_wave)
    run(std::true_type());
  else
    run(std::false_type());
  // dBias: the dBias pass's partial sums added up in increasing group order, as a
  // grid-stride pass of this grid once each workgroup's rows are done.
  if (dbias_part)
    dbias_reduce_range(dbias_part, dbias_groups, static_cast<int64_t>(p.H) * p.N * p.N, a.dbias,
                       static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x,
                       static_cast<int64_t>(gridDim.x) * kFThreads);
}

}  // namespace

bool bwd_fused_supported(const Problem& p) { return p.D <= 32 && p.N <= kFMaxKeys; }

hipError_t launch_bwd_fused(const Problem& p, const BwdArgs& a, const float* bias_k, const float* dbias_part,
                            int dbias_groups, hipStream_t s) {
  if (dbias_part && (a.dbias == nullptr || dbias_groups < 1 || dbias_groups > kMaxDbiasGroups))
    return hipErrorInvalidValue;
  // Persistent: one workgroup per compute unit (its LDS allows one).
  const int64_t blocks = std::min<int64_t>(static_cast<int64_t>(p.R) * p.H, device_cus());
  const int nt = bias_tiles(p.N);
  KernelTimer timer("bwd_fused_mfma", s);
  switch (p.D) {
    case 8:
      hipLaunchKernelGGL((bwd_fused_kernel<8>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt, dbias_part,
                         dbias_groups);
      break;
    case 16:
      hipLaunchKernelGGL((bwd_fused_kernel<16>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt, dbias_part,
                         dbias_groups);
      break;
    case 32:
      hipLaunchKernelGGL((bwd_fused_kernel<32>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt, dbias_part,
                         dbias_groups);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace evo
