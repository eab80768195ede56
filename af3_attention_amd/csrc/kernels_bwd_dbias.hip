// dBias of pair-biased 3D attention (bf16 MFMA, gfx950).
//
// The bias is shared by every attention row (MegaFold pages, gist.science
// technical summary, Methodik section 1 "EvoFlash-3D": an additively broadcast
// pair bias), so its gradient is a sum over rows:
//   dBias[h,j,k] = sum_r dS[r,h,j,k],  dS = P * (dP - D),
// with P recomputed from the saved logsumexp.  To make the sum deterministic,
// each workgroup owns a 128 x 128 (query x key) tile of one head and walks a
// fixed group of rows in increasing order, adding dS into registers; groups write
// partial sums that a last pass adds in increasing group order.
//
// Per row the workgroup stages Q, dO (its 128 queries), K, V (its 128 keys) and
// the row's pre-formed lse, D and mask operands in LDS with direct copies, through
// a ring of four stages (two at d = 64; copies run that many rows ahead minus
// one).  A wave owns 32 keys and one (d >= 32: 16 waves) or two (8 waves) 32-query
// tiles:
//   S  = Q K^T + sqrt(d) bias + sqrt(d) (mask - lse)   (bias: accumulator input;
//        mask and lse: one extra MFMA step on split-bf16 operands)
//   dP = dO V^T - D                                   (D: one extra MFMA step)
//   acc += exp2(S log2(e)/sqrt(d)) * dP               (one mul, one exp2, one FMA)

#include <algorithm>
#include <type_traits>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kDbT = 128;      // tile edge (queries and keys)
// Waves: 4 key tiles x 4 query tiles, one 32 x 32 tile each (four waves per SIMD
// hide more of each tile's dependency chain) for d >= 32; 4 key tiles x 2 query
// halves, two tiles each, at smaller d, where the shorter MFMA chains leave the
// exp work dominant and fewer waves with two independent tiles measured faster.
template <int D>
constexpr int db_tpw() { return D >= 32 ? 1 : 2; }  // query tiles per wave
template <int D>
constexpr int db_threads() { return 64 * 4 * (4 / db_tpw<D>()); }
// LDS ring of rows (copies run db_stages - 1 rows ahead): four stages of 38 KB
// up to d = 32, two of 70 KB at d = 64.
template <int D>
constexpr int db_stages() { return D >= 64 ? 2 : 4; }

template <int D>
__global__ __launch_bounds__(db_threads<D>(), 1) void dbias_pipe_kernel(Problem p, BwdArgs a,
                                                                   const float* __restrict__ bias_k, int nt,
                                                                   int groups, float* __restrict__ out) {
  constexpr int TB = Tile<D, kDbT>::BYTES;
  constexpr int STATS = 3 * kDbT * 16;  // query-side (lse, D; 32 B per query) and key-side (mask) operands
  constexpr int STAGE = 4 * TB + STATS;
  constexpr int NS = db_stages<D>();
  constexpr int DUMMY = NS * STAGE;  // 1 KB target of dummy copies
  constexpr int KS = Shape<D>::KS;
  constexpr int TPW = db_tpw<D>();
  using St = Stager<D, 2, kDbT, db_threads<D>()>;
  constexpr int NROW = 2 * St::NIT + 1;  // copies per thread per row: Q/dO, K/V, one operand piece
  __shared__ __align__(16) char lds[NS * STAGE + 1024];

  const int nb = (p.N + kDbT - 1) / kDbT;
  int blk = xcd_logical_block(blockIdx.x, nb * nb * groups * p.H);
  const int kb = blk % nb;
  blk /= nb;
  const int qb = blk % nb;
  blk /= nb;
  const int g = blk % groups;
  const int h = blk / groups;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wk = wave & 3, wq = wave >> 2;  // key tile, query group of this wave
  const int q0 = qb * kDbT, k0 = kb * kDbT;

  const int rows_per = (p.R + groups - 1) / groups;
  const int r_begin = g * rows_per;
  const int r_end = min(p.R, r_begin + rows_per);

  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t pstride = static_cast<uint32_t>(p.pos_stride * p.H * D * 2);
  const uint32_t lds0 = lds_addr(lds);
  St stager;
  stager.init(wave, lane, pstride);
  TileReads<D> rd;
  rd.init(lane);

  // sqrt(d) * bias of this wave's 32 keys and two 32-query tiles: constant over
  // the rows, so it is loaded once.
  f32x16 bias[TPW], acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    bias[t] = load_bias_tile(bias_k + bias_tile_offset(h, qb * 4 + TPW * wq + t, kb * 4 + wk, nt), lane);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  }
  const u32x4 dp_key = key_aug_unit(lane);
  const uint16_t* const qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* const dop = static_cast<const uint16_t*>(a.dout);
  const uint16_t* const kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* const vp = static_cast<const uint16_t*>(a.v);

  // Rows are issued in increasing order: running offsets of the next row to issue
  // (its Q/dO/K/V element offset, this wave's piece of its query operands, its key
  // operands).
  int64_t iss_rh = row_head_offset(p, r_begin, h);
  const int64_t rh_step = p.row_stride * p.H * D;
  const u32x4* iss_qo = static_cast<const u32x4*>(a.qops) +
                        2 * (static_cast<int64_t>(r_begin) * p.H + h) * qops_queries(p.N) + 2 * q0 + 64 * (wave & 3);
  const int64_t qo_step = 2 * static_cast<int64_t>(p.H) * qops_queries(p.N);
  const u32x4* iss_ka = static_cast<const u32x4*>(a.kaug) + static_cast<int64_t>(r_begin) * p.N;
  // Copies of the next row into stage s: Q, dO (queries q0..), K, V (keys k0..), and one
  // 64-entry piece of the split operands for each of waves 0..5: the 128 queries'
  // pre-formed operands (4 KB, waves 0..3) and the 128 keys' (2 KB, waves 4, 5).
  auto issue_row = [&](auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    const uint32_t st = lds0 + s * STAGE;
    const int64_t rh = iss_rh;
    iss_rh += rh_step;
    const char* qd[2] = {uniform_ptr(reinterpret_cast<const char*>(qp + rh)),
                         uniform_ptr(reinterpret_cast<const char*>(dop + rh))};
    const char* kv[2] = {uniform_ptr(reinterpret_cast<const char*>(kp + rh)),
                         uniform_ptr(reinterpret_cast<const char*>(vp + rh))};
    stager.issue(st, qd, q0, p.N, wave, lds0 + DUMMY);
    stager.issue(st + 2 * TB, kv, k0, p.N, wave, lds0 + DUMMY);
    const u32x4* const qo = iss_qo;
    const u32x4* const ka = iss_ka;
    iss_qo += qo_step;
    iss_ka += p.N;
    if (wave < 4) {
      copy16_to_lds(uniform_ptr(qo), static_cast<uint32_t>(lane) * 16, st + 4 * TB + 1024 * wave);
    } else if (wave < 6) {
      const int piece = wave & 1;
      copy_rows16(ka, k0 + 64 * piece, p.N, st + 4 * TB + 2 * kDbT * 16 + 1024 * piece, lane);
    } else {  // keep one operand copy per wave and row, so that waits can count them
      copy16_to_lds(uniform_ptr(a.kaug), 0u, lds0 + DUMMY);
    }
  };

  auto step = [&](int r, auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    // Row r was issued NS - 1 rows ago; up to NS - 2 later rows came after it.
    const int later = min(NS - 2, r_end - 1 - r);
    if (later >= 2)
      wait_vmcnt<2 * NROW>();
    else if (later == 1)
      wait_vmcnt<NROW>();
    else
      wait_vmcnt<0>();
    barrier();
    if (r + NS - 1 < r_end) issue_row(std::integral_constant<int, (s + NS - 1) % NS>());
    const uint32_t st = lds0 + s * STAGE;
    const uint32_t tq = st, tdo = st + TB, tk = st + 2 * TB, tv = st + 3 * TB;
    const uint32_t stats = st + 4 * TB;
    const int kl = wk * 32 + (lane & 31);  // this lane's key within the tile

    u32x4 s_key = lds_load16(stats + 2 * kDbT * 16 + kl * 16);
    u32x4 kop[KS], vop[KS];
    if constexpr (D == 8) {
      // The per-row terms ride in k slots 8..15 (lanes 32..63) of the one MFMA step.
      kop[0] = rd.rows_operand_with(tk, wk * 32, lane, s_key);
      vop[0] = rd.rows_operand_with(tv, wk * 32, lane, u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u});
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kop[ks] = rd.rows_operand(tk, wk * 32, ks, lane);
        vop[ks] = rd.rows_operand(tv, wk * 32, ks, lane);
      }
      if (lane >> 5) s_key = u32x4{0u, 0u, 0u, 0u};
    }

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int x0 = (TPW * wq + t) * 32;      // first query of this tile within the block
      const int jl = x0 + (lane & 31);       // this lane's query (as an A-operand row)
      const u32x4 s_q = lds_load16(stats + (jl >> 5) * 1024 + (jl & 31) * 16);
      const u32x4 dp_q = lds_load16(stats + (jl >> 5) * 1024 + 512 + (jl & 31) * 16);
      f32x16 sacc, dp;
      if constexpr (D == 8) {
        sacc = mma(rd.rows_operand_with(tq, x0, lane, s_q), kop[0], bias[t]);
        dp = mma(rd.rows_operand_with(tdo, x0, lane, dp_q), vop[0], f32x16{});
      } else {
        // Every operand read of the tile is issued before its first product (at
        // d = 64 the operands of both products would not fit in the registers).
        u32x4 qo[KS], dop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qo[ks] = rd.rows_operand(tq, x0, ks, lane);
          dop[ks] = rd.rows_operand(tdo, x0, ks, lane);
        }
        if constexpr (D <= 32) __builtin_amdgcn_sched_barrier(0);
        sacc = mma(qo[0], kop[0], bias[t]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) sacc = mma(qo[ks], kop[ks], sacc);
        sacc = mma(s_q, s_key, sacc);
        dp = mma(dop[0], vop[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) dp = mma(dop[ks], vop[ks], dp);
        dp = mma(dp_q, dp_key, dp);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = __builtin_fmaf(fast_exp2(sacc[e] * c1), dp[e], acc[t][e]);
    }
  };

  // Prologue: the bias tiles have arrived, then rows r_begin .. r_begin + NS - 2
  // go into stages 0 .. NS - 2.
#pragma unroll
  for (int t = 0; t < TPW; ++t) retire(bias[t]);
  if (r_begin < r_end) issue_row(std::integral_constant<int, 0>());
  if constexpr (NS > 2) {
    if (r_begin + 1 < r_end) issue_row(std::integral_constant<int, 1>());
    if (r_begin + 2 < r_end) issue_row(std::integral_constant<int, 2 % NS>());
  }
  for (int r = r_begin; r < r_end; r += NS) {
    step(r, std::integral_constant<int, 0>());
    if (r + 1 < r_end) step(r + 1, std::integral_constant<int, 1>());
    if constexpr (NS > 2) {
      if (r + 2 < r_end) step(r + 2, std::integral_constant<int, 2 % NS>());
      if (r + 3 < r_end) step(r + 3, std::integral_constant<int, 3 % NS>());
    }
  }

  // Partial sums of this group: out[g][h][j][k].
  const int key = k0 + wk * 32 + (lane & 31);
  if (key >= p.N) return;
  float* dst = out + (static_cast<int64_t>(g) * p.H + h) * p.N * p.N + key;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = q0 + (TPW * wq + t) * 32 + acc_row(v, lane);
      if (j < p.N) dst[static_cast<int64_t>(j) * p.N] = acc[t][v];
    }
}

}  // namespace

int dbias_pipe_groups(const Problem& p) {
  const int nb = (p.N + kDbT - 1) / kDbT;
  const int64_t tiles = static_cast<int64_t>(p.H) * nb * nb;
  // One workgroup per CU at a time (256 CUs on MI355X): pick the number of row
  // groups g <= 16 whose tiles * g workgroups fill the last round best (ties: the
  // smallest g, which also keeps the partial sums and their reduction small).
  constexpr int64_t kCus = 256;
  int best = 1;
  double best_eff = 0.0;
  for (int g = 1; g <= 16 && g <= p.R; ++g) {
    const int64_t wgs = tiles * g;
    const double eff = static_cast<double>(wgs) / static_cast<double>(kCus * ((wgs + kCus - 1) / kCus));
    if (eff > best_eff + 1e-3) {
      best_eff = eff;
      best = g;
    }
    if (eff >= 0.98) break;
  }
  return best;
}

hipError_t launch_dbias_pipe(const Problem& p, const BwdArgs& a, const float* bias_k, int groups, float* out,
                             hipStream_t s) {
  const int nb = (p.N + kDbT - 1) / kDbT;
  const int64_t blocks = static_cast<int64_t>(nb) * nb * groups * p.H;
  const int nt = bias_tiles(p.N);
  KernelTimer timer("bwd_dbias_mfma", s);
  switch (p.D) {
    case 8:
      hipLaunchKernelGGL((dbias_pipe_kernel<8>), dim3(blocks), dim3(db_threads<8>()), 0, s, p, a, bias_k, nt, groups, out);
      break;
    case 16:
      hipLaunchKernelGGL((dbias_pipe_kernel<16>), dim3(blocks), dim3(db_threads<16>()), 0, s, p, a, bias_k, nt, groups, out);
      break;
    case 32:
      hipLaunchKernelGGL((dbias_pipe_kernel<32>), dim3(blocks), dim3(db_threads<32>()), 0, s, p, a, bias_k, nt, groups, out);
      break;
    case 64:
      hipLaunchKernelGGL((dbias_pipe_kernel<64>), dim3(blocks), dim3(db_threads<64>()), 0, s, p, a, bias_k, nt, groups, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace evo
