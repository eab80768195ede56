// bf16 MFMA forward of pair-biased 3D attention for gfx950.
//
// The MegaFold pages (gist.science technical summary, Methodik section 1
// "EvoFlash-3D") describe the method: logits of a row are produced tile by tile
// in on-chip memory and normalised with an online, numerically stable softmax
// (Milakov and Gimelshein, "Online normalizer calculation for softmax"), so the
// R*H*N*N logit tensor never reaches HBM; the pair bias is added to every row.
//
// Mapping to CDNA4:
//  * one workgroup = 4 waves = 128 queries of one (row r, head h); each wave owns
//    32 queries and walks the keys in blocks of 64;
//  * the logits are produced transposed, S^T = K Q^T (keys x queries), so each
//    lane holds 32 keys of one query: the softmax max and sum over keys are
//    in-lane reductions plus one exchange with lane l ^ 32;
//  * the MFMA accumulator starts from sqrt(d) * (bias + mask) in fp32 (a
//    pre-pass writes the scaled bias once per call), so bias and mask cost no
//    vector ALU work; one FMA per logit applies log2(e)/sqrt(d) and subtracts
//    the running max before the exp2;
//  * P^T stays in registers and is, after packing to bf16, directly the B
//    operand of O^T = V^T P^T; V is staged transposed in LDS;
//  * key blocks whose keys are all masked are skipped; blocks with no masked
//    key skip the mask add.

#include <algorithm>

#include "mfma_common.h"

namespace evo {
namespace {

using namespace mfma;

constexpr int kFwdQueries = 128;  // queries per workgroup (32 per wave)
// Attention rows per wave; the rows of a wave share each load of the bias tile.
template <int D>
constexpr int fwd_rows() { return D <= 32 ? 2 : 1; }

// out[h][j][k] = sqrt(d) * bias[h][j][k] for j, k < N; -inf for k >= N (padding keys
// never win the softmax); 0 for padding queries.  Row stride nk, nq rows per head.
// transpose_out writes out[h][k][j] instead (the layout the backward's S tiles need).
template <typename T>
__global__ __launch_bounds__(256) void bias_prep_kernel(Problem p, const T* __restrict__ bias, float* __restrict__ out,
                                                        int nq, int nk, int transpose_out) {
  const int64_t total = static_cast<int64_t>(p.H) * nq * nk;
  const float sd = sqrtf(static_cast<float>(p.D));
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int inner = static_cast<int>(idx % nk);
    const int outer = static_cast<int>((idx / nk) % nq);
    const int h = static_cast<int>(idx / (static_cast<int64_t>(nk) * nq));
    const int j = transpose_out ? inner : outer;
    const int k = transpose_out ? outer : inner;
    float val;
    if (k >= p.N) {
      val = -INFINITY;
    } else if (j >= p.N || bias == nullptr) {
      val = 0.f;
    } else {
      val = sd * Elem<T>::load(bias, (static_cast<int64_t>(h) * p.N + j) * p.N + k);
    }
    out[idx] = val;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(Problem p, FwdArgs a, const float* __restrict__ bias_s,
                                                               int np) {
  using S = Shape<D>;
  constexpr int kFwdRows = fwd_rows<D>();
  constexpr int KROW = S::ROW;    // K rows, read as b128 operands
  constexpr int VROW = S::TRROW;  // V rows, read with transposing loads
  __shared__ __align__(16) uint16_t k_lds[2][kFwdRows][kStep * KROW];
  __shared__ __align__(16) uint16_t v_lds[2][kFwdRows][kStep * VROW];
  __shared__ __align__(16) float m_lds[2][kFwdRows][kStep];

  const int nqb = (p.N + kFwdQueries - 1) / kFwdQueries;
  int blk = blockIdx.x;
  const int qb = blk % nqb;
  blk /= nqb;
  const int h = blk % p.H;
  const int rp = blk / p.H;  // row group: rows kFwdRows * rp + i
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int j0 = qb * kFwdQueries + wave * 32;
  const int j = j0 + col;  // this lane's query (< np)
  const bool wave_active = j0 < p.N;

  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;
  const int64_t pstep = pos_step(p);

  int rr[kFwdRows];
  bool rvalid[kFwdRows];
  const uint16_t* kbase[kFwdRows];
  const uint16_t* vbase[kFwdRows];
  const float* mrow[kFwdRows];
  u32x4 qreg[kFwdRows][S::KS];
  f32x16 oacc[kFwdRows][S::DB];
  float m_run[kFwdRows], l_run[kFwdRows];
  Stage<D> kst[kFwdRows], vst[kFwdRows];
  float mnext[kFwdRows];
#pragma unroll
  for (int i = 0; i < kFwdRows; ++i) {
    rvalid[i] = kFwdRows * rp + i < p.R;
    rr[i] = rvalid[i] ? kFwdRows * rp + i : kFwdRows * rp;  // an invalid row aliases a valid one
    const int64_t rh = row_head_offset(p, rr[i], h);
    kbase[i] = static_cast<const uint16_t*>(a.k) + rh;
    vbase[i] = static_cast<const uint16_t*>(a.v) + rh;
    mrow[i] = a.mask ? a.mask + static_cast<int64_t>(rr[i]) * p.N : nullptr;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks)
      qreg[i][ks] = global_operand<D>(p, static_cast<const uint16_t*>(a.q), rr[i], j, h, ks, half);
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[i][db][e] = 0.f;
    m_run[i] = -INFINITY;  // running max of this query's logits, log2 units
    l_run[i] = 0.f;        // this lane's share of the running sum
    kst[i].init(p);
    vst[i].init(p);
    kst[i].load(kbase[i], 0, p.N);
    vst[i].load(vbase[i], 0, p.N);
    mnext[i] = mrow[i] ? mrow[i][min(lane, p.N - 1)] : 0.f;
  }

  // The scaled bias of the next block, shared by the rows of the group.
  const float* bhead = bias_s + static_cast<int64_t>(h) * np * np;  // uniform
  const uint32_t boff = static_cast<uint32_t>(j * np);              // per lane
  f32x16 bnext[2];
  bnext[0] = load_acc_rows(bhead + boff, half);
  bnext[1] = load_acc_rows(bhead + boff + 32, half);

  int buf = 0;
  for (int k0 = 0; k0 < p.N; k0 += kStep) {
    // Classify the block by its mask (the same in every wave of the workgroup).
    const bool valid = k0 + lane < p.N;
    bool any_mask[kFwdRows];
    float mv[kFwdRows];
    bool any_live = false;
#pragma unroll
    for (int i = 0; i < kFwdRows; ++i) {
      mv[i] = valid ? mnext[i] : 0.f;
      any_live = any_live || (rvalid[i] && __ballot(valid && mv[i] != -INFINITY) != 0);
      any_mask[i] = __ballot(mv[i] != 0.f) != 0;
    }
    const int k1 = k0 + kStep;
    if (!any_live) {  // every key of the block is masked in every row of the group
      if (k1 < p.N) {
#pragma unroll
        for (int i = 0; i < kFwdRows; ++i) {
          kst[i].load(kbase[i] + k1 * pstep, k1, p.N);
          vst[i].load(vbase[i] + k1 * pstep, k1, p.N);
          if (mrow[i]) mnext[i] = mrow[i][min(k1 + lane, p.N - 1)];
        }
        bnext[0] = load_acc_rows(bhead + k1 + boff, half);
        bnext[1] = load_acc_rows(bhead + k1 + boff + 32, half);
      }
      continue;
    }
    const int cb = buf;
#pragma unroll
    for (int i = 0; i < kFwdRows; ++i) {
      kst[i].store(k_lds[buf][i], nullptr, KROW, k0, p.N);
      vst[i].store(v_lds[buf][i], nullptr, VROW, k0, p.N);
      if (any_mask[i] && tid < kStep) m_lds[buf][i][tid] = valid ? sd * mv[i] : -INFINITY;
    }
    lds_barrier();
    buf ^= 1;

    // S^T tiles (keys k0 + 32 mb + ..., lane = query) of every row; the prefetched
    // sqrt(d) * bias registers are the first MFMA's accumulator input.
    f32x16 s[kFwdRows][2];
#pragma unroll
    for (int i = 0; i < kFwdRows; ++i) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 a0 = rows_operand<D>(k_lds[cb][i], mb * 32, 0, col, half);
        if (any_mask[i])
          s[i][mb] = mma(a0, qreg[i][0], bnext[mb] + load_acc_rows(&m_lds[cb][i][mb * 32], half));
        else
          s[i][mb] = mma(a0, qreg[i][0], bnext[mb]);
#pragma unroll
        for (int ks = 1; ks < S::KS; ++ks)
          s[i][mb] = mma(rows_operand<D>(k_lds[cb][i], mb * 32, ks, col, half), qreg[i][ks], s[i][mb]);
      }
    }

    // Prefetch the next block; overlaps the softmax and P V below.
    if (k1 < p.N) {
#pragma unroll
      for (int i = 0; i < kFwdRows; ++i) {
        kst[i].load(kbase[i] + k1 * pstep, k1, p.N);
        vst[i].load(vbase[i] + k1 * pstep, k1, p.N);
        if (mrow[i]) mnext[i] = mrow[i][min(k1 + lane, p.N - 1)];
      }
      bnext[0] = load_acc_rows(bhead + k1 + boff, half);
      bnext[1] = load_acc_rows(bhead + k1 + boff + 32, half);
    }

#pragma unroll
    for (int i = 0; i < kFwdRows; ++i) {
      // Online softmax over this block's keys (exp2 domain).  A row whose keys
      // are all masked so far keeps m = -inf; its exponent base is then 0, so
      // every P of the block is exp2(-inf) = 0.
      const float mx = pair_max(tile_max(s[i][0], s[i][1]));
      const float m_new = fmaxf(m_run[i], mx * c1);
      if (__ballot(m_new != m_run[i]) != 0) {  // some query's max grew: rescale
        const float alpha = fast_exp2(m_run[i] - m_new);
        l_run[i] *= alpha;
#pragma unroll
        for (int db = 0; db < S::DB; ++db) oacc[i][db] *= alpha;
      }
      m_run[i] = m_new;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;

      u32x4 pb[2][2];  // P^T packed to bf16: [key tile][16-key half]
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(s[i][mb][8 * t + e], c1, -m_use));
          pb[mb][t] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                            pack_bf16(pv[6], pv[7])};
        }
      }
      // Row sum of the bf16 probabilities that enter P V (four independent chains).
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) ls[e] = add_bf16_pair(pb[mb][t][e], ls[e]);
      l_run[i] += (ls[0] + ls[1]) + (ls[2] + ls[3]);

      // O^T += V^T P^T over the 64 keys (four 16-deep steps per 32-row block of d).
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            oacc[i][db] = mma(tr_operand<D>(v_lds[cb][i], VROW, db, mb * 32, t, lane), pb[mb][t], oacc[i][db]);
    }
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
hipError_t fwd_mfma_dispatch(const Problem& p, const FwdArgs& a, float* bias_s, int np, hipStream_t s) {
  hipError_t e = launch_bias_prep(p, a.bias, bias_s, np, 0, s);
  if (e != hipSuccess) return e;
  constexpr int rows = fwd_rows<D>();
  const int64_t blocks =
      static_cast<int64_t>((p.N + kFwdQueries - 1) / kFwdQueries) * p.H * ((p.R + rows - 1) / rows);
  KernelTimer timer("fwd_mfma", s);
  hipLaunchKernelGGL((fwd_mfma_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, p, a,
                     bias_s, np);
  return hipGetLastError();
}

}  // namespace

int bias_pad(int n) { return (n + 127) / 128 * 128; }

hipError_t launch_bias_prep(const Problem& p, const void* bias, float* out, int np, int transpose_out,
                            hipStream_t s) {
  const int64_t total = static_cast<int64_t>(p.H) * np * np;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 8192));
  KernelTimer timer(transpose_out ? "bias_prep_t" : "bias_prep", s);
  hipLaunchKernelGGL((bias_prep_kernel<uint16_t>), dim3(blocks), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), out, np, np, transpose_out);
  return hipGetLastError();
}

size_t fwd_mfma_workspace_bytes(const Problem& p) {
  const int64_t np = bias_pad(p.N);
  return static_cast<size_t>(p.H) * np * np * sizeof(float);
}

hipError_t launch_fwd_mfma(const Problem& p, const FwdArgs& a, void* ws, hipStream_t s) {
  const int np = bias_pad(p.N);
  float* bias_s = static_cast<float*>(ws);
  switch (p.D) {
    case 8: return fwd_mfma_dispatch<8>(p, a, bias_s, np, s);
    case 16: return fwd_mfma_dispatch<16>(p, a, bias_s, np, s);
    case 32: return fwd_mfma_dispatch<32>(p, a, bias_s, np, s);
    case 64: return fwd_mfma_dispatch<64>(p, a, bias_s, np, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evo
