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
//  * 12 waves; wave w owns the 32 keys 32 w .. 32 w + 31 (waves past the keys
//    have no tile) and keeps their dK, dV in registers while the workgroup walks
//    the queries in blocks of 32.  Q, dO and the per-query split operands of a
//    block are staged in LDS by direct copies, double buffered; the row's K is
//    staged once and stays;
//  * tiles are S = Q K^T (queries x keys), so a lane holds one key:
//      S  = Q K^T + sqrt(d) bias + sqrt(d) (mask - lse)   (bias: accumulator input,
//           a tiled fp32 copy loaded one block ahead; mask and lse: one extra
//           MFMA step on split-bf16 operands)
//      dP = dO V^T - D                                   (D: one extra MFMA step)
//      P = exp2(S log2(e)/sqrt(d)),  dS = P dP
//    P and dS, packed to bf16 in registers, are the B operands of dV^T += dO^T P
//    and dK^T += Q^T dS (A operands: transposing LDS reads of dO and Q);
//  * each wave also writes its dS tile to LDS as [key][query]; during the next
//    block waves 0..3 each form one 16 x 16 quadrant of dQ^T for the finished
//    query tile, sum over all key tiles, with v_mfma_f32_16x16x32_bf16 (one
//    instruction per 32-key tile; A = K^T and B = dS^T from transposing LDS
//    reads), and store it.  The dS tiles are double buffered, so one barrier
//    per block orders everything.

#include <algorithm>
#include <type_traits>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kFw = 12;               // waves per workgroup (one 32-key tile each)
constexpr int kFThreads = 64 * kFw;
constexpr int kFMaxKeys = 32 * kFw;   // keys per row this kernel handles
constexpr int kFq = 32;               // queries per block
constexpr int kDsBytes = 32 * 64;     // one dS tile: 32 keys x 32 queries, bf16

typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kFThreads, 1) void bwd_fused_kernel(Problem p, BwdArgs a,
                                                                  const float* __restrict__ bias_k, int nt) {
  constexpr int KS = Shape<D>::KS;
  static_assert(Shape<D>::DB == 1, "head_dim <= 32");
  constexpr int TQ = Tile<D, kFq>::BYTES;   // one staged tile of 32 queries
  constexpr int STAGE = 2 * TQ + 1024;      // Q, dO, query-side operands (64 entries)
  constexpr int KRES = kFMaxKeys * 2 * D;   // the row's K
  using StQ = Stager<D, 2, kFq, kFThreads>;
  using StK = Stager<D, 1, kFMaxKeys, kFThreads>;
  __shared__ __align__(16) char lds[KRES + 2 * STAGE + 2 * kFw * kDsBytes + 1024];
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t k_res = lds0;
  const uint32_t stage0 = lds0 + KRES;
  const uint32_t ds0 = stage0 + 2 * STAGE;
  const uint32_t dummy = ds0 + 2 * kFw * kDsBytes;

  // Workgroups of one head are contiguous per XCD (its L2 then holds that head's
  // bias tiles).
  const int logical = xcd_logical_block(blockIdx.x, p.R * p.H);
  const int h = logical / p.R, r = logical % p.R;
  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int nkt = (p.N + 31) / 32;  // key tiles = query blocks
  const bool tile_wave = wave < nkt;
  const int key = wave * 32 + (lane & 31);
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t pstride = static_cast<uint32_t>(p.pos_stride * p.H * D * 2);

  StQ stq;
  stq.init(wave, lane, pstride);
  StK stk;
  stk.init(wave, lane, pstride);
  TileReads<D> rd;
  rd.init(lane);

  const uint16_t* const qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* const dop = static_cast<const uint16_t*>(a.dout);
  const uint16_t* const kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* const vp = static_cast<const uint16_t*>(a.v);
  const int64_t rh = row_head_offset(p, r, h);

  // V of this lane's key (B operand; K's comes from the staged row) and the
  // key-side split operand.
  u32x4 vop[KS], s_key = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) vop[ks] = u32x4{0u, 0u, 0u, 0u};
  if (tile_wave) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) vop[ks] = global_operand<D>(p, vp, r, key, h, ks, half);
    s_key = static_cast<const u32x4*>(a.kaug)[static_cast<int64_t>(r) * p.N + min(key, p.N - 1)];
  }
  if (half) s_key = u32x4{0u, 0u, 0u, 0u};
  const u32x4 dp_key = key_aug_unit(lane);
  f32x16 dk_acc, dv_acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) dk_acc[e] = dv_acc[e] = 0.f;

  const char* const qbase[2] = {uniform_ptr(reinterpret_cast<const char*>(qp + rh)),
                                uniform_ptr(reinterpret_cast<const char*>(dop + rh))};
  const char* const kbase[1] = {uniform_ptr(reinterpret_cast<const char*>(kp + rh))};
  const u32x4* const qaug_row =
      uniform_ptr(static_cast<const u32x4*>(a.qaug) + (static_cast<int64_t>(r) * p.H + h) * p.N);

  // Copies of query block b (Q, dO, and the query-side operands by the last wave).
  auto issue_block = [&](int b, uint32_t st) __attribute__((always_inline)) {
    stq.issue(st, qbase, b * kFq, p.N, wave, dummy);
    if (wave == kFw - 1) copy_rows16(qaug_row, b * kFq, p.N, st + 2 * TQ, lane);
  };
  // sqrt(d) * bias of this wave's keys for the 32 queries of block b.
  auto load_bias = [&](f32x16& dst, int b) __attribute__((always_inline)) {
    if (tile_wave) dst = load_bias_tile(bias_k + bias_tile_offset(h, b, wave, nt), lane);
  };

  // dQ: wave w < 4 forms the quadrant d0 = 16 (w & 1), queries q0 = 16 (w >> 1)
  // of dQ^T of a finished query tile (d0 >= D: nothing to form).
  const int dq_d0 = 16 * (wave & 1), dq_q0 = 16 * (wave >> 1);
  const bool dq_wave = wave < 4 && dq_d0 < D;
  const int g4 = lane >> 4, i16 = lane & 15;
  int ca = dq_d0 + 4 * (i16 & 3);
  if (ca >= D) ca &= (D - 1);  // channels >= D only feed rows that are never stored
  const int offA0 = Tile<D>::quad_off(8 * g4 + (i16 >> 2), ca);
  const int offA1 = Tile<D>::quad_off(8 * g4 + 4 + (i16 >> 2), ca);
  const int offB0 = Tile<32>::quad_off(8 * g4 + (i16 >> 2), dq_q0 + 4 * (i16 & 3));
  const int offB1 = Tile<32>::quad_off(8 * g4 + 4 + (i16 >> 2), dq_q0 + 4 * (i16 & 3));
  auto dq_tile = [&](int qb, uint32_t dsbuf) __attribute__((always_inline)) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt < nkt; ++kt) {
      const uint32_t ka = k_res + kt * (32 * 2 * D);
      const uint32_t da = dsbuf + kt * kDsBytes;
      const u32x2 a0 = lds_load_tr(ka + offA0), a1 = lds_load_tr(ka + offA1);
      const u32x2 b0 = lds_load_tr(da + offB0), b1 = lds_load_tr(da + offB1);
      acc = mma16(u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{b0[0], b0[1], b1[0], b1[1]}, acc);
    }
    // lane: query q0 + (lane & 15), channels d0 + 4 (lane >> 4) + 0..3
    const int q = qb * kFq + dq_q0 + i16;
    const int d = dq_d0 + 4 * g4;
    if (q < p.N && d < D) {
      const float s = 1.f / sd;
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dq) + elem_offset(p, r, q, h) + d) =
          u32x2{pack_bf16(acc[0] * s, acc[1] * s), pack_bf16(acc[2] * s, acc[3] * s)};
    }
  };

  // One 32 x 32 score tile of block b: this wave's keys, the block's queries.
  auto tile_row = [&](int b, uint32_t st, const f32x16& bias, uint32_t dsw) __attribute__((always_inline)) {
    const uint32_t tq = st, tdo = st + TQ;
    const int jl = lane & 31;
    const u32x4 qa = lds_load16(st + 2 * TQ + jl * 16);
    const u32x4 s_q =
        b * kFq + jl < p.N ? u32x4{qa[0], qa[1], kBf16One | (kBf16One << 16), 0u} : dead_query_aug();
    const u32x4 dp_q = {qa[2], qa[3], 0u, 0u};
    const uint32_t kt_lds = k_res + wave * (32 * 2 * D);  // this wave's keys in the staged row
    f32x16 sacc = mma(rd.rows_operand(tq, 0, 0, lane), rd.rows_operand(kt_lds, 0, 0, lane), bias);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
      sacc = mma(rd.rows_operand(tq, 0, ks, lane), rd.rows_operand(kt_lds, 0, ks, lane), sacc);
    sacc = mma(s_q, s_key, sacc);
    f32x16 dp = mma(rd.rows_operand(tdo, 0, 0, lane), vop[0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) dp = mma(rd.rows_operand(tdo, 0, ks, lane), vop[ks], dp);
    dp = mma(dp_q, dp_key, dp);

    u32x4 pb[2], dsb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(sacc[8 * u + e] * c1);
        dsv[e] = pv[e] * dp[8 * u + e];
      }
      pb[u] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                    pack_bf16(pv[6], pv[7])};
      dsb[u] = u32x4{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                     pack_bf16(dsv[6], dsv[7])};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      dv_acc = mma(rd.tr_operand(tdo, 0, 0, u), pb[u], dv_acc);
      dk_acc = mma(rd.tr_operand(tq, 0, 0, u), dsb[u], dk_acc);
    }
    // dS to LDS as [key][query]: registers 8u .. 8u + 3 hold queries 16 u + 4 half
    // + 0..3, registers 8u + 4 .. 8u + 7 hold queries 16 u + 8 + 4 half + 0..3.
    const int x = lane & 31;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 4 * half)) = u32x2{dsb[u][0], dsb[u][1]};
      *reinterpret_cast<lds_u32x2*>(dsw + Tile<32>::quad_off(x, 16 * u + 8 + 4 * half)) =
          u32x2{dsb[u][2], dsb[u][3]};
    }
  };

  f32x16 bias[2];
  // Block b: everything issued one block earlier has arrived and every wave has
  // finished block b - 1 (its stage and its dS buffer are complete; the buffers of
  // block b - 2 are free).  Block b + 1's copies and bias start at once.
  auto step = [&](int b, auto s_c) __attribute__((always_inline)) {
    constexpr int s = decltype(s_c)::value;
    wait_vmcnt<0>();
    barrier();
    retire(bias[s]);
    if (b + 1 < nkt) {
      issue_block(b + 1, stage0 + (s ^ 1) * STAGE);
      load_bias(bias[s ^ 1], b + 1);
    }
    if (dq_wave && b > 0) dq_tile(b - 1, ds0 + (s ^ 1) * (kFw * kDsBytes));
    if (tile_wave) tile_row(b, stage0 + s * STAGE, bias[s], ds0 + s * (kFw * kDsBytes) + wave * kDsBytes);
  };

  // Prologue: the operands loaded above arrive before any copy is issued.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) retire(vop[ks]);
  retire(s_key);
  stk.issue(k_res, kbase, 0, p.N, wave, dummy);
  issue_block(0, stage0);
  load_bias(bias[0], 0);
  for (int b = 0; b < nkt; b += 2) {
    step(b, std::integral_constant<int, 0>());
    if (b + 1 < nkt) step(b + 1, std::integral_constant<int, 1>());
  }
  wait_vmcnt<0>();
  barrier();
  if (dq_wave) dq_tile(nkt - 1, ds0 + ((nkt - 1) & 1) * (kFw * kDsBytes));

  if (!tile_wave || key >= p.N) return;
  const int64_t off = elem_offset(p, r, key, h);
  store_dT<D>(static_cast<uint16_t*>(a.dv) + off, &dv_acc, 1.f, half);
  store_dT<D>(static_cast<uint16_t*>(a.dk) + off, &dk_acc, 1.f / sd, half);
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
