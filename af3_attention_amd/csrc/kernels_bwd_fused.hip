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
// A workgroup owns one attention row r of one head h and all its keys, so every
// sum above completes inside it and nothing is accumulated across workgroups:
//  * 8 waves, two per SIMD.  The 12 key tiles of 32 keys are split so that each
//    SIMD carries three: wave w < 4 owns tiles w and w + 4, wave w >= 4 owns tile
//    w + 4 and also forms dQ (below).  Each wave keeps its tiles' dK, dV in
//    registers while the workgroup walks the queries in blocks of 32.  The row's K
//    and V are staged in LDS once; Q, dO and the per-query split operands of each
//    block are staged by direct copies, double buffered;
//  * tiles are S = Q K^T (queries x keys), so a lane holds one key:
//      S  = Q K^T + sqrt(d) bias + sqrt(d) (mask - lse)   (bias: accumulator input,
//           a tiled fp32 copy loaded one block ahead; mask and lse: one extra
//           MFMA step on split-bf16 operands)
//      dP = dO V^T - D                                   (D: one extra MFMA step)
//      P = exp2(S log2(e)/sqrt(d)),  dS = P dP
//    P and dS, packed to bf16 in registers, are the B operands of dV^T += dO^T P
//    and dK^T += Q^T dS (A operands: transposing LDS reads of dO and Q); the two
//    tiles of a wave w < 4 are independent work the compiler interleaves;
//  * each tile's dS goes to LDS as [key][query].  During the next block wave
//    w >= 4 forms quadrant w - 4 (16 channels x 16 queries) of dQ^T of the
//    finished query tile over all key tiles with v_mfma_f32_16x16x32_bf16, one
//    instruction per 32-key tile (A = K^T and B = dS^T from transposing LDS
//    reads), and stores it.  The dS tiles are double buffered, so one barrier per
//    block orders everything.

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

__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Per key tile of a wave: the key-side split operand, the dK^T and dV^T
// accumulators and the bias of the current and the next block.
struct KeyTile {
  int kt;       // key tile index
  bool valid;   // kt < number of key tiles of the row
  u32x4 s_key;
  f32x16 dk, dv;
  f32x16 bias[2];
};

template <int D>
__global__ __launch_bounds__(kFThreads, 1) void bwd_fused_kernel(Problem p, BwdArgs a,
                                                                  const float* __restrict__ bias_k, int nt) {
  constexpr int KS = Shape<D>::KS;
  static_assert(Shape<D>::DB == 1, "head_dim <= 32");
  constexpr int TQ = Tile<D, kFq>::BYTES;   // one staged tile of 32 queries
  constexpr int STAGE = 2 * TQ + 1024;      // Q, dO, query-side operands (64 entries)
  constexpr int KRES = kFMaxKeys * 2 * D;   // the row's K (and then its V)
  using StQ = Stager<D, 2, kFq, kFThreads>;
  using StK = Stager<D, 2, kFMaxKeys, kFThreads>;
  __shared__ __align__(16) char lds[2 * KRES + 2 * STAGE + 2 * kFTiles * kDsBytes + 1024];
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t k_res = lds0, v_res = lds0 + KRES;
  const uint32_t stage0 = lds0 + 2 * KRES;
  const uint32_t ds0 = stage0 + 2 * STAGE;
  const uint32_t dummy = ds0 + 2 * kFTiles * kDsBytes;

  // Workgroups of one head are contiguous per XCD (its L2 then holds that head's
  // bias tiles).
  const int logical = xcd_logical_block(blockIdx.x, p.R * p.H);
  const int h = logical / p.R, r = logical % p.R;
  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int nkt = (p.N + 31) / 32;  // key tiles = query blocks
  const bool pair_wave = wave < 4;  // two key tiles; otherwise one tile and dQ
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t pstride = static_cast<uint32_t>(p.pos_stride * p.H * D * 2);

  TileReads<D> rd;
  rd.init(lane);

  const uint16_t* const qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* const dop = static_cast<const uint16_t*>(a.dout);
  const uint16_t* const kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* const vp = static_cast<const uint16_t*>(a.v);
  const int64_t rh = row_head_offset(p, r, h);

  // Tile A: w (w < 4) or w + 4; tile B: w + 4 (w < 4 only).  Invalid tiles (past
  // the row's keys) run on clamped, finite data and are never stored.
  KeyTile ta, tb;
  ta.kt = pair_wave ? wave : wave + 4;
  tb.kt = wave + 4;
  ta.valid = ta.kt < nkt;
  tb.valid = pair_wave && tb.kt < nkt;
  auto init_tile = [&](KeyTile& t) __attribute__((always_inline)) {
    const int key = min(t.kt * 32 + (lane & 31), p.N - 1);
    t.s_key = static_cast<const u32x4*>(a.kaug)[static_cast<int64_t>(r) * p.N + key];
    if (half) t.s_key = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) t.dk[e] = t.dv[e] = 0.f;
  };
  init_tile(ta);
  if (pair_wave) init_tile(tb);

  const char* const qbase[2] = {uniform_ptr(reinterpret_cast<const char*>(qp + rh)),
                                uniform_ptr(reinterpret_cast<const char*>(dop + rh))};
  const char* const kvbase[2] = {uniform_ptr(reinterpret_cast<const char*>(kp + rh)),
                                 uniform_ptr(reinterpret_cast<const char*>(vp + rh))};
  const u32x4* const qaug_row =
      uniform_ptr(static_cast<const u32x4*>(a.qaug) + (static_cast<int64_t>(r) * p.H + h) * p.N);

  // Copies of query block b (Q, dO, and the query-side operands by the last wave).
  auto issue_block = [&](int b, uint32_t st) __attribute__((always_inline)) {
    // The per-lane copy offsets are recomputed here rather than kept live across
    // the loop (the empty asm keeps the compiler from hoisting them).
    int l = lane;
    asm volatile("" : "+v"(l));
    StQ stq;
    stq.init(wave, l, pstride);
    stq.issue(st, qbase, b * kFq, p.N, wave, dummy);
    if (wave == kFw - 1) copy_rows16(qaug_row, b * kFq, p.N, st + 2 * TQ, l);
  };
  // sqrt(d) * bias of tile t's keys for the 32 queries of block b.
  auto load_bias = [&](const KeyTile& t, f32x16& dst, int b) __attribute__((always_inline)) {
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
  // The quadrant for query block qb, whose dS tiles are in buffer dsbuf: a sum over
  // the row's key tiles, reads issued four tiles at a time.
  auto dq_tile = [&](int qb, uint32_t dsbuf) __attribute__((always_inline)) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto product = [&](int kt) __attribute__((always_inline)) {
      const uint32_t ka = k_res + kt * (32 * 2 * D), da = dsbuf + kt * kDsBytes;
      const u32x2 a0 = lds_load_tr(ka + offA0), a1 = lds_load_tr(ka + offA1);
      const u32x2 b0 = lds_load_tr(da + offB0), b1 = lds_load_tr(da + offB1);
      return std::make_pair(u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{b0[0], b0[1], b1[0], b1[1]});
    };
    int kt = 0;
    for (; kt + 4 <= nkt; kt += 4) {
      const auto o0 = product(kt), o1 = product(kt + 1), o2 = product(kt + 2), o3 = product(kt + 3);
      acc = mma16(o0.first, o0.second, acc);
      acc = mma16(o1.first, o1.second, acc);
      acc = mma16(o2.first, o2.second, acc);
      acc = mma16(o3.first, o3.second, acc);
    }
    for (; kt < nkt; ++kt) {
      const auto o = product(kt);
      acc = mma16(o.first, o.second, acc);
    }
    // lane: query q0 + (lane & 15), channels d0 + 4 (lane >> 4) + 0..3
    const int q = qb * kFq + dq_q0 + i16;
    const int d = dq_d0 + 4 * g4;
    if (q < p.N && d < D) {
      const float sc = 1.f / sd;
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dq) + elem_offset(p, r, q, h) + d) =
          u32x2{pack_bf16(acc[0] * sc, acc[1] * sc), pack_bf16(acc[2] * sc, acc[3] * sc)};
    }
  };

  // Score tile (block b, key tile t), in three phases: (1) S and dP on the matrix
  // cores, (2) P and dS on the vector ALU, (3) dV, dK on the matrix cores and dS
  // into the dS buffer.
  struct Scores {
    f32x16 s, dp;
  };
  struct Probs {
    u32x4 p[2], ds[2];
  };
  auto phase1 = [&](int b, uint32_t st, const KeyTile& t, const f32x16& bias) __attribute__((always_inline)) {
    const uint32_t tq = st, tdo = st + TQ;
    const int jl = lane & 31;
    const u32x4 qa = lds_load16(st + 2 * TQ + jl * 16);
    const u32x4 s_q =
        b * kFq + jl < p.N ? u32x4{qa[0], qa[1], kBf16One | (kBf16One << 16), 0u} : dead_query_aug();
    const u32x4 dp_q = {qa[2], qa[3], 0u, 0u};
    const uint32_t kt_lds = k_res + t.kt * (32 * 2 * D), vt_lds = v_res + t.kt * (32 * 2 * D);
    Scores o;
    o.s = mma(rd.rows_operand(tq, 0, 0, lane), rd.rows_operand(kt_lds, 0, 0, lane), bias);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      o.s = mma(rd.rows_operand(tq, 0, ks, lane), rd.rows_operand(kt_lds, 0, ks, lane), o.s);
    o.s = mma(s_q, t.s_key, o.s);
    o.dp = mma(rd.rows_operand(tdo, 0, 0, lane), rd.rows_operand(vt_lds, 0, 0, lane), f32x16{});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      o.dp = mma(rd.rows_operand(tdo, 0, ks, lane), rd.rows_operand(vt_lds, 0, ks, lane), o.dp);
    // (the key side of the D step is rebuilt here rather than kept live)
    int l = lane;
    asm volatile("" : "+v"(l));
    o.dp = mma(dp_q, key_aug_unit(l), o.dp);
    return o;
  };
  auto phase2 = [&](const Scores& sc) __attribute__((always_inline)) {
    Probs o;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(sc.s[8 * u + e] * c1);
        dsv[e] = pv[e] * sc.dp[8 * u + e];
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
    const uint32_t dsw = dsbuf + min(t.kt, kFTiles - 1) * kDsBytes;
    const int x = lane & 31;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 4 * half)) =
          u32x2{pr.ds[u][0], pr.ds[u][1]};
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 8 + 4 * half)) =
          u32x2{pr.ds[u][2], pr.ds[u][3]};
    }
  };
  auto tile_row = [&](int b, uint32_t st, KeyTile& t, const f32x16& bias, uint32_t dsbuf)
                      __attribute__((always_inline)) { phase3(st, t, phase2(phase1(b, st, t, bias)), dsbuf); };

  // Block b: everything issued one block earlier has arrived and every wave has
  // finished block b - 1 (its stage and its dS tiles are complete; the buffers of
  // block b - 2 are free).  Block b + 1's copies and bias start at once.  The two
  // roles run separate copies of the loop (the same number of barriers), so that
  // neither role's registers have to be reconciled with the other's.
  auto step = [&](int b, auto s_c, auto pair_c) __attribute__((always_inline)) {
    constexpr int s = decltype(s_c)::value;
    constexpr bool PAIR = decltype(pair_c)::value;
    wait_vmcnt<0>();
    barrier();
    retire(ta.bias[s]);
    if constexpr (PAIR) retire(tb.bias[s]);
    if (b + 1 < nkt) {
      issue_block(b + 1, stage0 + (s ^ 1) * STAGE);
      load_bias(ta, ta.bias[s ^ 1], b + 1);
      if constexpr (PAIR) load_bias(tb, tb.bias[s ^ 1], b + 1);
    }
    const uint32_t st = stage0 + s * STAGE, dsb = ds0 + s * (kFTiles * kDsBytes);
    if constexpr (PAIR) {
      tile_row(b, st, ta, ta.bias[s], dsb);
      tile_row(b, st, tb, tb.bias[s], dsb);
    } else {
      if (dq_wave && b >= 1) dq_tile(b - 1, ds0 + (s ^ 1) * (kFTiles * kDsBytes));
      tile_row(b, st, ta, ta.bias[s], dsb);
    }
  };
  auto run = [&](auto pair_c) __attribute__((always_inline)) {
    constexpr bool PAIR = decltype(pair_c)::value;
    load_bias(ta, ta.bias[0], 0);
    if constexpr (PAIR) load_bias(tb, tb.bias[0], 0);
    for (int b = 0; b < nkt; b += 2) {
      step(b, std::integral_constant<int, 0>(), pair_c);
      if (b + 1 < nkt) step(b + 1, std::integral_constant<int, 1>(), pair_c);
    }
    wait_vmcnt<0>();
    barrier();
    if constexpr (!PAIR) {
      if (dq_wave) dq_tile(nkt - 1, ds0 + ((nkt - 1) & 1) * (kFTiles * kDsBytes));
    }
  };

  // Prologue: the operands loaded above arrive before any copy is issued.
  retire(ta.s_key);
  if (pair_wave) retire(tb.s_key);
  {
    StK stk;
    stk.init(wave, lane, pstride);
    stk.issue(k_res, kvbase, 0, p.N, wave, dummy);
  }
  issue_block(0, stage0);
  if (pair_wave)
    run(std::true_type());
  else
    run(std::false_type());

  auto store_tile = [&](const KeyTile& t) __attribute__((always_inline)) {
    const int key = t.kt * 32 + (lane & 31);
    if (!t.valid || key >= p.N) return;
    const int64_t off = elem_offset(p, r, key, h);
    store_dT<D>(static_cast<uint16_t*>(a.dv) + off, &t.dv, 1.f, half);
    store_dT<D>(static_cast<uint16_t*>(a.dk) + off, &t.dk, 1.f / sd, half);
  };
  store_tile(ta);
  if (pair_wave) store_tile(tb);
}

}  // namespace

bool bwd_fused_supported(const Problem& p) { return p.D <= 32 && p.N <= kFMaxKeys; }

hipError_t launch_bwd_fused(const Problem& p, const BwdArgs& a, const float* bias_k, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.R) * p.H;
  const int nt = bias_tiles(p.N);
  KernelTimer timer("bwd_fused_mfma", s);
  switch (p.D) {
    case 8: hipLaunchKernelGGL((bwd_fused_kernel<8>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt); break;
    case 16: hipLaunchKernelGGL((bwd_fused_kernel<16>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt); break;
    case 32: hipLaunchKernelGGL((bwd_fused_kernel<32>), dim3(blocks), dim3(kFThreads), 0, s, p, a, bias_k, nt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace evo
