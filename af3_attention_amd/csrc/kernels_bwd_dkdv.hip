// dK and dV of pair-biased 3D attention (bf16 MFMA, gfx950).
//
// The backward recomputes the probabilities from the saved logsumexp instead of
// storing them (the pages' memory-efficient kernel runs in the forward and the
// backward: gist.science MegaFold technical summary, Methodik section 1
// "EvoFlash-3D").  With dS = P * (dP - D):
//   dV[k] = sum_j P[j,k] dO[j],   dK[k] = sum_j dS[j,k] Q[j] / sqrt(d).
//
// Workgroup = 4 waves = 128 keys of two rows (r, r+1) of one head (one row at
// d = 64); wave w owns the 32 keys 32 w.. of both rows, so each bias tile it
// loads serves two rows, and keeps their dK, dV in registers while it walks all
// queries in blocks of 64.  Q, dO and the rows' per-query split operands are
// staged in LDS with direct copies, double buffered, and shared by the four
// waves.  Tiles are S = Q K^T (queries x keys), so each lane holds one key:
//   S  = Q K^T + sqrt(d) bias + sqrt(d) (mask - lse)   (bias: accumulator input,
//        loaded a block ahead into alternating registers; mask and lse: one
//        extra MFMA step)
//   dP = dO V^T - D                                   (D: one extra MFMA step)
//   P = exp2(S log2(e)/sqrt(d)),  dS = P dP
// and P, dS in registers, packed to bf16, are directly the B operands of
// dV^T += dO^T P and dK^T += Q^T dS, whose A operands come from transposing LDS
// reads of the staged dO and Q.

#include <algorithm>
#include <type_traits>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kKvKeys = 128;  // keys per workgroup (32 per wave)
// Attention rows per workgroup (and per wave): two, or one at d = 64 where two
// rows' operands and accumulators would not fit the registers.
template <int D>
constexpr int kv_rows() { return D >= 64 ? 1 : 2; }

template <int D>
__global__ __launch_bounds__(256, 2) void dkdv_pipe_kernel(Problem p, BwdArgs a, const float* __restrict__ bias_k,
                                                           int nt) {
  constexpr int RW = kv_rows<D>();
  constexpr int TB = Tile<D>::BYTES;               // 64 queries
  constexpr int NT = 2 * RW;                       // Q, dO of each row
  constexpr int STAGE = NT * TB + RW * kBlk * 16;  // + query-side operands
  constexpr int KS = Shape<D>::KS, DB = Shape<D>::DB;
  using St = Stager<D, NT>;
  __shared__ __align__(16) char lds[2 * STAGE + 1024];
  constexpr int DUMMY = 2 * STAGE;

  const int nkb = (p.N + kKvKeys - 1) / kKvKeys;
  const int nrp = (p.R + RW - 1) / RW;
  int blk = xcd_logical_block(blockIdx.x, nkb * nrp * p.H);
  const int kb = blk % nkb;
  blk /= nkb;
  const int rp = blk % nrp;
  const int h = blk / nrp;
  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int k0w = kb * kKvKeys + wave * 32;  // first key of this wave
  const int key = k0w + (lane & 31);         // this lane's key
  const bool wave_active = k0w < p.N;
  const int nqb = (p.N + kBlk - 1) / kBlk;

  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const uint32_t lds0 = lds_addr(lds);
  St stager;
  stager.init(wave, lane, static_cast<uint32_t>(p.pos_stride * p.H * D * 2));
  TileReads<D> rd;
  rd.init(lane);

  // Per row: K and V of this lane's key (B operands), the key-side split
  // operands, dK^T and dV^T accumulators.
  bool rvalid[RW];
  int rr[RW];
  u32x4 kop[RW][KS], vop[RW][KS], s_key[RW];
  f32x16 dk_acc[RW][DB], dv_acc[RW][DB];
  const char* base[NT];
  const u32x4* qaug_row[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    rvalid[i] = RW * rp + i < p.R;
    rr[i] = rvalid[i] ? RW * rp + i : RW * rp;  // an invalid row aliases a valid one
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kop[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.k), rr[i], key, h, ks, half);
      vop[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.v), rr[i], key, h, ks, half);
    }
    s_key[i] = static_cast<const u32x4*>(a.kaug)[static_cast<int64_t>(rr[i]) * p.N + min(key, p.N - 1)];
    if (half) s_key[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dk_acc[i][db][e] = dv_acc[i][db][e] = 0.f;
    // Staged per block: Q r0, dO r0, Q r1, dO r1, then the query-side operands of
    // both rows (64 entries of 16 bytes each).
    const int64_t rh = row_head_offset(p, rr[i], h);
    base[2 * i] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.q) + rh));
    base[2 * i + 1] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.dout) + rh));
    qaug_row[i] = uniform_ptr(static_cast<const u32x4*>(a.qaug) + (static_cast<int64_t>(rr[i]) * p.H + h) * p.N);
  }
  const u32x4 dp_key = key_aug_unit(lane);

  auto issue_block = [&](int qb, auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    const uint32_t st = lds0 + s * STAGE;
    stager.issue(st, base, qb * kBlk, p.N, wave, lds0 + DUMMY);
    if (wave < RW)
      copy_rows16(wave == 0 ? qaug_row[0] : qaug_row[RW - 1], qb * kBlk, p.N, st + NT * TB + wave * kBlk * 16, lane);
    else
      copy16_to_lds(uniform_ptr(qaug_row[0]), 0u, lds0 + DUMMY);
  };

  // sqrt(d) * bias of the wave's keys for 32-query tile t of block qb.
  const int kt = min(kb * (kKvKeys / 32) + wave, nt - 1);
  auto load_bias = [&](f32x16& b, int qb, int t) {
    b = load_bias_tile(bias_k + bias_tile_offset(h, 2 * qb + t, kt, nt), lane);
  };
  // One register tile per query tile: tile t of block qb + 1 is loaded as soon as
  // both rows of block qb have used tile t.
  f32x16 bias[2];

  auto step = [&](int qb, auto stage_c) {
    constexpr int s = decltype(stage_c)::value;
    // Block qb's copies and bias tiles were the last memory operations issued.
    wait_vmcnt<0>();
    barrier();
    // (Tell the compiler the bias tiles have arrived, before the copies below:
    // its own wait for them would otherwise also drain those copies.)
    retire(bias[0]);
    retire(bias[1]);
    // Start block qb + 1's copies at once into the other buffer (read during the
    // previous block).
    if (qb + 1 < nqb) issue_block(qb + 1, std::integral_constant<int, s ^ 1>());
    if (!wave_active) return;
    const uint32_t st = lds0 + s * STAGE;

#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const uint32_t tq = st + (2 * i) * TB, tdo = st + (2 * i + 1) * TB;
        const uint32_t qaug_lds = st + NT * TB + i * kBlk * 16;
        const int jl = t * 32 + (lane & 31);
        const u32x4 qa = lds_load16(qaug_lds + jl * 16);
        const u32x4 s_q = qb * kBlk + jl < p.N ? u32x4{qa[0], qa[1], kBf16One | (kBf16One << 16), 0u}
                                               : dead_query_aug();
        const u32x4 dp_q = {qa[2], qa[3], 0u, 0u};
        f32x16 sacc = mma(rd.rows_operand(tq, t * 32, 0, lane), kop[i][0], bias[t]);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) sacc = mma(rd.rows_operand(tq, t * 32, ks, lane), kop[i][ks], sacc);
        sacc = mma(s_q, s_key[i], sacc);
        // (the last block reloads its own tiles: a harmless, branch-free extra load)
        if (i == RW - 1) load_bias(bias[t], min(qb + 1, nqb - 1), t);
        f32x16 dp = mma(rd.rows_operand(tdo, t * 32, 0, lane), vop[i][0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) dp = mma(rd.rows_operand(tdo, t * 32, ks, lane), vop[i][ks], dp);
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
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            dv_acc[i][db] = mma(rd.tr_operand(tdo, db, t * 32, u), pb[u], dv_acc[i][db]);
            dk_acc[i][db] = mma(rd.tr_operand(tq, db, t * 32, u), dsb[u], dk_acc[i][db]);
          }
      }
    }
  };

  // The operands loaded above have arrived before the loop issues its copies.
#pragma unroll
  for (int i = 0; i < RW; ++i) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      retire(kop[i][ks]);
      retire(vop[i][ks]);
    }
    retire(s_key[i]);
  }
  load_bias(bias[0], 0, 0);
  load_bias(bias[1], 0, 1);
  issue_block(0, std::integral_constant<int, 0>());
  for (int qb = 0; qb < nqb; qb += 2) {
    step(qb, std::integral_constant<int, 0>());
    if (qb + 1 < nqb) step(qb + 1, std::integral_constant<int, 1>());
  }

  if (!wave_active || key >= p.N) return;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (!rvalid[i]) continue;
    const int64_t off = elem_offset(p, rr[i], key, h);
    store_dT<D>(static_cast<uint16_t*>(a.dv) + off, dv_acc[i], 1.f, half);
    store_dT<D>(static_cast<uint16_t*>(a.dk) + off, dk_acc[i], 1.f / sd, half);
  }
}

}  // namespace

hipError_t launch_dkdv_pipe(const Problem& p, const BwdArgs& a, const float* bias_k, hipStream_t s) {
  const int rows = p.D >= 64 ? kv_rows<64>() : kv_rows<32>();
  const int64_t blocks = static_cast<int64_t>((p.N + kKvKeys - 1) / kKvKeys) * p.H * ((p.R + rows - 1) / rows);
  const int nt = bias_tiles(p.N);
  KernelTimer timer("bwd_dkdv_mfma", s);
  switch (p.D) {
    case 8: hipLaunchKernelGGL((dkdv_pipe_kernel<8>), dim3(blocks), dim3(256), 0, s, p, a, bias_k, nt); break;
    case 16: hipLaunchKernelGGL((dkdv_pipe_kernel<16>), dim3(blocks), dim3(256), 0, s, p, a, bias_k, nt); break;
    case 32: hipLaunchKernelGGL((dkdv_pipe_kernel<32>), dim3(blocks), dim3(256), 0, s, p, a, bias_k, nt); break;
    case 64: hipLaunchKernelGGL((dkdv_pipe_kernel<64>), dim3(blocks), dim3(256), 0, s, p, a, bias_k, nt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace evo
