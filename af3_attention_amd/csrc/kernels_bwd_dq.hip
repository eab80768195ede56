// dQ of pair-biased 3D attention (bf16 MFMA, gfx950).
//
// The backward recomputes the probabilities from the saved logsumexp (MegaFold
// pages, gist.science technical summary, Methodik section 1 "EvoFlash-3D": the
// memory-efficient kernel runs in the forward and the backward).  With
// dS = P * (dP - D):  dQ[j] = sum_k dS[j,k] K[k] / sqrt(d).
//
// Workgroup = 4 waves = 128 queries of two rows (r, r+1) of one head (one row at
// d = 64); wave w owns the 32 queries 32 w.. of both rows, so each bias tile it
// loads serves two rows, and keeps their dQ in registers while it walks all keys
// in blocks of 64.  K, V and the rows' per-key split operands are staged in LDS
// with direct copies, double buffered, and shared by the four waves.  Tiles are S^T = K Q^T (keys x
// queries), so each lane holds one query:
//   S^T  = K Q^T + sqrt(d) bias^T + sqrt(d) (mask - lse)  (bias: accumulator
//          input, loaded a block ahead; mask and lse: one extra MFMA step)
//   dP^T = V dO^T - D                                    (D: one extra MFMA step)
//   P = exp2(S log2(e)/sqrt(d)),  dS = P dP
// and dS^T in registers, packed to bf16, is directly the B operand of
// dQ^T += K^T dS^T, whose A operand comes from transposing LDS reads of K.

#include <algorithm>
#include <type_traits>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kDqQueries = 128;  // queries per workgroup (32 per wave)
// Attention rows per workgroup (and per wave): two, or one at d = 64 where two
// rows' operands and accumulators would not fit the registers.
template <int D>
constexpr int dq_rows() { return D >= 64 ? 1 : 2; }

template <int D>
__global__ __launch_bounds__(256, 2) void dq_pipe_kernel(Problem p, BwdArgs a, const float* __restrict__ bias_q,
                                                         int nt) {
  constexpr int kDqRows = dq_rows<D>();
  // Software-pipelined units where the registers allow it (not at d = 64).
  constexpr bool kPipelined = D <= 32;
  constexpr int TB = Tile<D>::BYTES;                    // 64 keys
  constexpr int NT = 2 * kDqRows;                       // K, V of each row
  constexpr int STAGE = NT * TB + kDqRows * kBlk * 16;  // + key-side operands
  constexpr int KS = Shape<D>::KS, DB = Shape<D>::DB;
  using St = Stager<D, NT>;
  __shared__ __align__(16) char lds[2 * STAGE + 1024];
  constexpr int DUMMY = 2 * STAGE;

  const int nqb = (p.N + kDqQueries - 1) / kDqQueries;
  const int nrp = (p.R + kDqRows - 1) / kDqRows;
  int blk = xcd_logical_block(blockIdx.x, nqb * nrp * p.H);
  const int qb = blk % nqb;
  blk /= nqb;
  const int rp = blk % nrp;
  const int h = blk / nrp;
  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int j0 = qb * kDqQueries + wave * 32;
  const int j = j0 + (lane & 31);  // this lane's query
  const bool wave_active = j0 < p.N;
  const int nkb = (p.N + kBlk - 1) / kBlk;

  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t lds0 = lds_addr(lds);
  St stager;
  stager.init(wave, lane, static_cast<uint32_t>(p.pos_stride * p.H * D * 2));
  TileReads<D> rd;
  rd.init(lane);

  // Per row: Q and dO of this lane's query (B operands), the query-side split
  // operands, the dQ^T accumulator.
  bool rvalid[kDqRows];
  int rr[kDqRows];
  u32x4 qop[kDqRows][KS], doop[kDqRows][KS], s_q[kDqRows], dp_q[kDqRows];
  f32x16 dq_acc[kDqRows][DB];
  const char* base[NT];
  const u32x4* kaug_row[kDqRows];
#pragma unroll
  for (int i = 0; i < kDqRows; ++i) {
    rvalid[i] = kDqRows * rp + i < p.R;
    rr[i] = rvalid[i] ? kDqRows * rp + i : kDqRows * rp;  // an invalid row aliases a valid one
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.q), rr[i], j, h, ks, half);
      doop[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.dout), rr[i], j, h, ks, half);
    }
    const u32x4 qa =
        static_cast<const u32x4*>(a.qaug)[(static_cast<int64_t>(rr[i]) * p.H + h) * p.N + min(j, p.N - 1)];
    s_q[i] = u32x4{qa[0], qa[1], kBf16One | (kBf16One << 16), 0u};
    dp_q[i] = u32x4{qa[2], qa[3], 0u, 0u};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq_acc[i][db][e] = 0.f;
    // Staged per block: K r0, V r0, K r1, V r1, then the key-side operands of both
    // rows (64 entries of 16 bytes each).
    const int64_t rh = row_head_offset(p, rr[i], h);
    base[2 * i] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k) + rh));
    base[2 * i + 1] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v) + rh));
    kaug_row[i] = uniform_ptr(static_cast<const u32x4*>(a.kaug) + static_cast<int64_t>(rr[i]) * p.N);
  }
  const u32x4 dp_key = key_aug_unit(lane);

  auto issue_block = [&](int kb, auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    const uint32_t st = lds0 + s * STAGE;
    stager.issue(st, base, kb * kBlk, p.N, wave, lds0 + DUMMY);
    if (wave < kDqRows)
      copy_rows16(wave == 0 ? kaug_row[0] : kaug_row[kDqRows - 1], kb * kBlk, p.N, st + NT * TB + wave * kBlk * 16,
                  lane);
    else
      copy16_to_lds(uniform_ptr(kaug_row[0]), 0u, lds0 + DUMMY);
  };

  // sqrt(d) * bias^T of the wave's queries for 32-key tile mb of block kb.
  const int qt = min(qb * (kDqQueries / 32) + wave, nt - 1);
  auto load_bias = [&](f32x16& b, int kb, int mb) {
    b = load_bias_tile(bias_q + bias_tile_offset(h, qt, 2 * kb + mb, nt), lane);
  };
  // One register tile per key tile: tile mb of block kb + 1 is loaded as soon as
  // every row of block kb has used tile mb.
  f32x16 bias[2];

  // A block is U = 2 * kDqRows units (key tile mb = u / kDqRows, row i = u % kDqRows),
  // each in three phases: A = LDS operand reads and the S^T, dP^T MFMAs; B = the
  // vector work giving dS^T; C = the dQ^T MFMAs.  Unit u's B and C phases run
  // beside unit u + 1's A phase, with LDS reads one unit further ahead; the
  // scheduling barriers keep each unit's group in this order.
  constexpr int U = 2 * kDqRows;
  struct AOps {
    u32x4 k[KS], v[KS], kaug;
  };
  struct COps {
    u32x4 kt[DB][2];
  };
  auto load_a = [&](AOps& o, uint32_t st, int u) {
    const int mb = u / kDqRows, i = u % kDqRows;
    const uint32_t tk = st + (2 * i) * TB, tv = st + (2 * i + 1) * TB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      o.k[ks] = rd.rows_operand(tk, mb * 32, ks, lane);
      o.v[ks] = rd.rows_operand(tv, mb * 32, ks, lane);
    }
    o.kaug = lds_load16(st + NT * TB + i * kBlk * 16 + (mb * 32 + (lane & 31)) * 16);
  };
  auto load_c = [&](COps& o, uint32_t st, int u) {
    const int mb = u / kDqRows, i = u % kDqRows;
    const uint32_t tk = st + (2 * i) * TB;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) o.kt[db][t] = rd.tr_operand(tk, db, mb * 32, t);
  };
  auto phase_a = [&](const AOps& o, int kb, int u, f32x16& sacc, f32x16& dp) {
    const int mb = u / kDqRows, i = u % kDqRows;
    const u32x4 s_key = half ? u32x4{0u, 0u, 0u, 0u} : o.kaug;
    sacc = mma(o.k[0], qop[i][0], bias[mb]);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) sacc = mma(o.k[ks], qop[i][ks], sacc);
    sacc = mma(s_key, s_q[i], sacc);
    // (the last block reloads its own tile: a harmless, branch-free extra load)
    if (i == kDqRows - 1) load_bias(bias[mb], min(kb + 1, nkb - 1), mb);
    dp = mma(o.v[0], doop[i][0], f32x16{});
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) dp = mma(o.v[ks], doop[i][ks], dp);
    dp = mma(dp_key, dp_q[i], dp);
  };
  auto phase_bc = [&](const COps& o, int u, const f32x16& sacc, const f32x16& dp) {
    const int i = u % kDqRows;
    u32x4 dsb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsv[e] = fast_exp2(sacc[8 * t + e] * c1) * dp[8 * t + e];
      dsb[t] = u32x4{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                     pack_bf16(dsv[6], dsv[7])};
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) dq_acc[i][db] = mma(o.kt[db][t], dsb[t], dq_acc[i][db]);
  };

  auto step = [&](int kb, auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    // Block kb's copies and bias tiles were the last memory operations issued.
    wait_vmcnt<0>();
    barrier();
    // (Tell the compiler the bias tiles have arrived, before the copies below:
    // its own wait for them would otherwise also drain those copies.)
    retire(bias[0]);
    retire(bias[1]);
    // Start block kb + 1's copies at once into the other buffer (read during the
    // previous block).
    if (kb + 1 < nkb) issue_block(kb + 1, std::integral_constant<int, s ^ 1>());
    if (!wave_active) return;
    const uint32_t st = lds0 + s * STAGE;

    if constexpr (kPipelined) {
      AOps ao[2];
      COps co[2];
      f32x16 sacc[2], dp[2];
      load_a(ao[0], st, 0);
      load_c(co[0], st, 0);
      if (U > 1) load_a(ao[1], st, 1);
      phase_a(ao[0], kb, 0, sacc[0], dp[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u + 1 < U) {
          load_c(co[(u + 1) & 1], st, u + 1);
          if (u + 2 < U) load_a(ao[u & 1], st, u + 2);
          phase_a(ao[(u + 1) & 1], kb, u + 1, sacc[(u + 1) & 1], dp[(u + 1) & 1]);
        }
        phase_bc(co[u & 1], u, sacc[u & 1], dp[u & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        AOps ao;
        COps co;
        f32x16 sacc, dp;
        load_a(ao, st, u);
        phase_a(ao, kb, u, sacc, dp);
        load_c(co, st, u);
        phase_bc(co, u, sacc, dp);
      }
    }
  };

  // The operands loaded above have arrived before the loop issues its copies.
#pragma unroll
  for (int i = 0; i < kDqRows; ++i) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      retire(qop[i][ks]);
      retire(doop[i][ks]);
    }
    retire(s_q[i]);
    retire(dp_q[i]);
  }
  load_bias(bias[0], 0, 0);
  load_bias(bias[1], 0, 1);
  issue_block(0, std::integral_constant<int, 0>());
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, std::integral_constant<int, 0>());
    if (kb + 1 < nkb) step(kb + 1, std::integral_constant<int, 1>());
  }

  if (!wave_active || j >= p.N) return;
#pragma unroll
  for (int i = 0; i < kDqRows; ++i)
    if (rvalid[i])
      store_dT<D>(static_cast<uint16_t*>(a.dq) + elem_offset(p, rr[i], j, h), dq_acc[i], 1.f / sd, half);
}

}  // namespace

hipError_t launch_dq_pipe(const Problem& p, const BwdArgs& a, const float* bias_q, hipStream_t s) {
  const int rows = p.D >= 64 ? dq_rows<64>() : dq_rows<32>();
  const int64_t blocks = static_cast<int64_t>((p.N + kDqQueries - 1) / kDqQueries) * p.H * ((p.R + rows - 1) / rows);
  const int nt = bias_tiles(p.N);
  KernelTimer timer("bwd_dq_mfma", s);
  switch (p.D) {
    case 8: hipLaunchKernelGGL((dq_pipe_kernel<8>), dim3(blocks), dim3(256), 0, s, p, a, bias_q, nt); break;
    case 16: hipLaunchKernelGGL((dq_pipe_kernel<16>), dim3(blocks), dim3(256), 0, s, p, a, bias_q, nt); break;
    case 32: hipLaunchKernelGGL((dq_pipe_kernel<32>), dim3(blocks), dim3(256), 0, s, p, a, bias_q, nt); break;
    case 64: hipLaunchKernelGGL((dq_pipe_kernel<64>), dim3(blocks), dim3(256), 0, s, p, a, bias_q, nt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace evo
