// bf16 MFMA forward of pair-biased 3D attention for gfx950, head_dim 64 (head_dim
// 8, 16 and 32 run the ping-pong kernel in kernels_fwd_pp.hip).
//
// The MegaFold pages (gist.science technical summary, Methodik section 1
// "EvoFlash-3D") describe the method: logits of a row are produced tile by tile
// in on-chip memory and normalised with an online, numerically stable softmax
// (Milakov and Gimelshein, "Online normalizer calculation for softmax"), so the
// R*H*N*N logit tensor never reaches HBM; the pair bias is added to every row.
//
// Mapping to CDNA4:
//  * one workgroup = 4 waves = 128 queries of two rows (r, r+1) of one head; each
//    wave owns 32 queries of both rows, so every bias tile it loads serves two rows;
//  * keys are walked in blocks of 64 through a four-stage LDS ring filled by
//    direct global -> LDS copies (no register staging) two blocks ahead, with one
//    workgroup barrier per block;
//  * the logits are produced transposed, S^T = K Q^T (keys x queries), so each lane
//    holds 32 keys of one query: the softmax max and sum are in-lane reductions
//    plus one exchange with lane l ^ 32;
//  * the softmax keeps a lazily refreshed reference point (the exponentials of a
//    block may exceed 1 until a lane's block sum crosses a bound), so a block
//    normally costs one FMA, one exp2, half a pack and one add per logit (the
//    normaliser sums the fp32 probabilities) and no max reduction or rescale;
//  * the MFMA accumulator starts from sqrt(d) * bias, read as four coalesced 1 KB
//    loads from a pre-pass's tiled copy, so the bias costs no vector ALU work;
//    one FMA per logit applies log2(e)/sqrt(d) and subtracts the running max;
//  * P^T stays in registers and, packed to bf16, is directly the B operand of
//    O^T = V^T P^T; V^T comes from transposing LDS reads (ds_read_b64_tr_b16);
//  * key blocks whose keys are all masked in both rows are skipped; blocks with no
//    masked key skip the mask add.
//  * workgroups are mapped so that each XCD works on one contiguous range of
//    (head, row pair) and its L2 holds one head's bias and the rows' K, V.

#include <algorithm>
#include <type_traits>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace pipe;

constexpr int kFwdQueries = 128;  // queries per workgroup (32 per wave)
constexpr int kFwdRows = 2;       // attention rows per workgroup
constexpr int kStages = 4;  // LDS ring of K/V stages (copies run two blocks ahead)

// Largest of the 32 values of two accumulator tiles (v_max3 chains; inputs are
// finite or -inf, never NaN).
__device__ __forceinline__ float max_of_tiles(const f32x16& a, const f32x16& b) {
  float m[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    m[u] = max3f(a[4 * u], a[4 * u + 1], a[4 * u + 2]);
    m[u] = max3f(m[u], a[4 * u + 3], b[4 * u]);
    m[u] = max3f(m[u], b[4 * u + 1], b[4 * u + 2]);
    m[u] = max3f(m[u], b[4 * u + 3], b[4 * u + 3]);
  }
  return max3f(m[0], m[1], max3f(m[2], m[3], m[3]));
}

__device__ __forceinline__ float pair_max_raw(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// A block's probabilities may exceed 1 by up to this factor before the running
// maximum is refreshed (the normalised result does not depend on the reference
// point; fp32 and bf16 keep the full range).
constexpr float kLazyMaxSum = 1048576.f;  // 2^20, bound on one lane's 32-term block sum

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_pipe_kernel(Problem p, FwdArgs a, const float* __restrict__ bias_t,
                                                          int nt) {
  constexpr int TB = Tile<D>::BYTES;
  constexpr int NT = 2 * kFwdRows;  // staged tiles per stage: K, V of each row
  constexpr int STAGE = NT * TB;
  using St = Stager<D, NT>;
  constexpr int NDMA = St::NIT;
  constexpr int KS = Shape<D>::KS, DB = Shape<D>::DB;
  __shared__ __align__(16) char lds[kStages * STAGE];
  __shared__ __align__(16) float mlds[kStages][kFwdRows][kBlk];

  const int nqb = (p.N + kFwdQueries - 1) / kFwdQueries;
  const int nrg = (p.R + kFwdRows - 1) / kFwdRows;
  int blk = xcd_logical_block(blockIdx.x, nqb * nrg * p.H);
  const int qb = blk % nqb;
  blk /= nqb;
  const int rg = blk % nrg;
  const int h = blk / nrg;
  const int wave = wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  const int j0 = qb * kFwdQueries + wave * 32;
  const int j = j0 + (lane & 31);  // this lane's query
  const bool wave_active = j0 < p.N;
  const int nkb = (p.N + kBlk - 1) / kBlk;

  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;

  int rr[kFwdRows];
  bool rvalid[kFwdRows];
  const char* tbase[NT];  // K r0, V r0, K r1, V r1
  const float* mrow[kFwdRows];
  u32x4 qreg[kFwdRows][KS];
  f32x16 oacc[kFwdRows][DB];
  float m_run[kFwdRows], l_run[kFwdRows];
#pragma unroll
  for (int i = 0; i < kFwdRows; ++i) {
    rvalid[i] = kFwdRows * rg + i < p.R;
    rr[i] = rvalid[i] ? kFwdRows * rg + i : kFwdRows * rg;  // an invalid row aliases a valid one
    const int64_t rh = row_head_offset(p, rr[i], h);
    tbase[2 * i] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.k) + rh));
    tbase[2 * i + 1] = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.v) + rh));
    mrow[i] = a.mask ? uniform_ptr(a.mask + static_cast<int64_t>(rr[i]) * p.N) : nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.q), rr[i], j, h, ks, half);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[i][db][e] = 0.f;
    m_run[i] = -INFINITY;  // reference point of this query's exponentials, log2 units
    l_run[i] = 0.f;        // this lane's share of the running sum
  }
  const bool masked = a.mask != nullptr;
  const uint32_t lds0 = lds_addr(lds), mlds0 = lds_addr(mlds);
  St stager;
  stager.init(wave, lane, static_cast<uint32_t>(p.pos_stride * p.H * D * 2));
  TileReads<D> rd;
  rd.init(lane);

  // Bias tiles of this wave's 32 queries: tile (qt, kt) of head h.
  const int qt = qb * (kFwdQueries / 32) + wave;
  const float* btile = bias_t + bias_tile_offset(h, min(qt, nt - 1), 0, nt);
  f32x16 bias_reg[2][2];  // two register sets: block kb uses set kb % 2, loaded two blocks ahead

  // Copies of stage kb % kStages: K and V of both rows, and (waves 0 and 1) the
  // mask of row `wave` for the block's 64 keys (keys >= N read key N - 1).
  auto issue_stage = [&](int kb, auto stage_c) {
    constexpr int sn = decltype(stage_c)::value;
    stager.issue(lds0 + sn * STAGE, tbase, kb * kBlk, p.N, wave);
    if (masked && wave < kFwdRows) {
      const uint32_t dst = mlds0 + (sn * kFwdRows + wave) * kBlk * 4;
      const float* m = wave == 0 ? mrow[0] : mrow[1];
      if (kb * kBlk + kBlk <= p.N)
        copy4_to_lds(uniform_ptr(m + kb * kBlk), static_cast<uint32_t>(lane) * 4, dst);
      else
        copy4_to_lds(m + min(kb * kBlk + lane, p.N - 1), dst);
    }
  };

  auto load_bias = [&](f32x16 (&dst)[2], int kb) {
    dst[0] = load_bias_tile(btile + (2 * kb) * 1024, lane);
    dst[1] = load_bias_tile(btile + (2 * kb + 1) * 1024, lane);
  };

  // Prologue: the query operands have arrived (so that no wait for them lands in
  // the loop), then bias and stage of blocks 0 and 1, in the order of the loop body.
#pragma unroll
  for (int i = 0; i < kFwdRows; ++i)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) retire(qreg[i][ks]);
  load_bias(bias_reg[0], 0);
  issue_stage(0, std::integral_constant<int, 0>());
  if (nkb > 1) {
    load_bias(bias_reg[1], 1);
    issue_stage(1, std::integral_constant<int, 1>());
  }

  // One block of 64 keys; its stage index is a compile-time constant (the loop
  // below is unrolled by kStages) so every LDS address is a fixed offset.
  auto step = [&](auto stage_c, int kb) {
    constexpr int st = decltype(stage_c)::value;
    // Stage kb was issued two blocks ago; after it this wave issued the bias
    // loads (8) and the stage of block kb + 1, if there is one.
    if (kb + 1 < nkb)
      wait_vmcnt<8 + NDMA>();
    else
      wait_vmcnt<0>();
    barrier();
    // Tell the compiler this block's bias registers have arrived: its own wait for
    // them, placed at their first use, would count only the loads it knows of and
    // so also drain the copies in flight.
    retire(bias_reg[st % 2][0]);
    retire(bias_reg[st % 2][1]);
    uint32_t kt_lds[kFwdRows], vt_lds[kFwdRows];
#pragma unroll
    for (int i = 0; i < kFwdRows; ++i) {
      kt_lds[i] = lds0 + st * STAGE + (2 * i) * TB;
      vt_lds[i] = lds0 + st * STAGE + (2 * i + 1) * TB;
    }

    // Classify the block by its mask (identical in every wave); keys >= N are dead.
    bool any_mask[kFwdRows];
    bool any_live = !masked;
    const bool kvalid = kb * kBlk + lane < p.N;
    if (masked) {
#pragma unroll
      for (int i = 0; i < kFwdRows; ++i) {
        const float mv = mlds[st][i][lane];
        any_mask[i] = __ballot(kvalid && mv != 0.f) != 0;
        any_live = any_live || (rvalid[i] && __ballot(kvalid && mv != -INFINITY) != 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kFwdRows; ++i) any_mask[i] = false;
    }
    const bool compute = any_live && wave_active;
    f32x16 (&bcur)[2] = bias_reg[st % 2];

    // S^T tiles (keys 32 mb + .., lane = query) of both rows; the bias registers
    // are the first MFMA's accumulator input.
    f32x16 s[kFwdRows][2];
    if (compute) {
#pragma unroll
      for (int i = 0; i < kFwdRows; ++i) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4 a0 = rd.rows_operand(kt_lds[i], mb * 32, 0, lane);
          if (any_mask[i])
            s[i][mb] = mma(a0, qreg[i][0], bcur[mb] + sd * lds_acc_rows(mlds0 + ((st * kFwdRows + i) * kBlk + mb * 32) * 4, half));
          else
            s[i][mb] = mma(a0, qreg[i][0], bcur[mb]);
#pragma unroll
          for (int ks = 1; ks < KS; ++ks)
            s[i][mb] = mma(rd.rows_operand(kt_lds[i], mb * 32, ks, lane), qreg[i][ks], s[i][mb]);
        }
      }
    }

    // A skipped block still retires its bias loads here, so that every path
    // reaches the next loads with no outstanding write to the bias registers.
    if (!compute) asm volatile("" ::"v"(bcur[0]), "v"(bcur[1]));

    // Prefetch block kb + 2: its bias into the registers block kb just used, then
    // its stage (that buffer was last read in iteration kb - 2).  Bias loads go
    // first, so that the compiler's wait for them at block kb + 2 leaves the
    // stage of block kb + 3 in flight.
    if (kb + 2 < nkb) {
      load_bias(bcur, kb + 2);
      issue_stage(kb + 2, std::integral_constant<int, (st + 2) % kStages>());
    }

    if (compute) {
#pragma unroll
      for (int i = 0; i < kFwdRows; ++i) {
        // Online softmax (exp2 domain) with a lazily refreshed reference point m:
        // P = exp2(S c1 - m).  While m is finite and no lane's 32-term block sum
        // exceeds kLazyMaxSum, the block is accumulated against the current m; else
        // m moves to the running maximum and the accumulators are rescaled.  A row
        // whose keys are all masked so far keeps m = -inf and gets P = 0.
        u32x4 pb[2][2];  // P^T packed to bf16: [key tile][16-key half]
        float lsum;
        auto exponentiate = [&](float m_use) {
          // The normaliser sums the fp32 probabilities (four independent chains).
          float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              float pv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                pv[e] = fast_exp2(__builtin_fmaf(s[i][mb][8 * t + e], c1, -m_use));
                ls[e & 3] += pv[e];
              }
              pb[mb][t] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                                pack_bf16(pv[6], pv[7])};
            }
          }
          lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        };
        const bool fresh = __ballot(m_run[i] == -INFINITY) != 0;
        if (!fresh) exponentiate(m_run[i]);
        if (fresh || __ballot(!(lsum <= kLazyMaxSum)) != 0) {
          const float mx = pair_max_raw(max_of_tiles(s[i][0], s[i][1])) * c1;
          const float m_new = fmaxf(m_run[i], mx);
          const float alpha = m_run[i] == -INFINITY ? 0.f : fast_exp2(m_run[i] - m_new);
          l_run[i] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[i][db] *= alpha;
          m_run[i] = m_new;
          exponentiate(m_new == -INFINITY ? 0.f : m_new);
        }
        l_run[i] += lsum;

        // O^T += V^T P^T over the 64 keys (four 16-deep steps per 32-row block of d).
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              oacc[i][db] = mma(rd.tr_operand(vt_lds[i], db, mb * 32, t), pb[mb][t], oacc[i][db]);
      }
    }
  };


  for (int kb = 0; kb < nkb; kb += kStages) {
    step(std::integral_constant<int, 0>(), kb);
    if (kb + 1 < nkb) step(std::integral_constant<int, 1>(), kb + 1);
    if (kb + 2 < nkb) step(std::integral_constant<int, 2>(), kb + 2);
    if (kb + 3 < nkb) step(std::integral_constant<int, 3>(), kb + 3);
  }

  if (!wave_active) return;
#pragma unroll
  for (int i = 0; i < kFwdRows; ++i) {
    const float l_tot = pair_sum(l_run[i]);
    if (j >= p.N || !rvalid[i]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    store_dT<D>(static_cast<uint16_t*>(a.o) + elem_offset(p, rr[i], j, h), oacc[i], inv, half);
    if (a.lse && half == 0)
      a.lse[(static_cast<int64_t>(rr[i]) * p.H + h) * p.N + j] =
          l_tot > 0.f ? (m_run[i] + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t fwd_pipe_dispatch(const Problem& p, const FwdArgs& a, float* bias_t, hipStream_t s) {
  hipError_t e = launch_bias_tiles(p, a.bias, bias_t, nullptr, s);
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>((p.N + kFwdQueries - 1) / kFwdQueries) * p.H *
                         ((p.R + kFwdRows - 1) / kFwdRows);
  KernelTimer timer("fwd_mfma", s);
  hipLaunchKernelGGL((fwd_pipe_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, a, bias_t,
                     bias_tiles(p.N));
  return hipGetLastError();
}

}  // namespace

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Workspace: tiled bias | (head_dim <= 32) per-key mask operands [R,N] x 16 B |
// last live key of each row [R] x 4 B.
size_t fwd_mfma_workspace_bytes(const Problem& p) {
  size_t b = align256(tiled_bias_bytes(p));
  if (p.D <= 32) b += align256(static_cast<size_t>(p.R) * p.N * 16) + align256(static_cast<size_t>(p.R) * 4);
  return b;
}

hipError_t launch_fwd_mfma(const Problem& p, const FwdArgs& a, void* ws, hipStream_t s) {
  float* bias_t = static_cast<float*>(ws);
  if (p.D <= 32) {
    char* kaug = static_cast<char*>(ws) + align256(tiled_bias_bytes(p));
    int* last_live = reinterpret_cast<int*>(kaug + align256(static_cast<size_t>(p.R) * p.N * 16));
    return launch_fwd_pp(p, a, bias_t, kaug, last_live, s);
  }
  switch (p.D) {
    case 64: return fwd_pipe_dispatch<64>(p, a, bias_t, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evo
