// bf16 MFMA backward of pair-biased 3D attention for gfx950.
//
// The backward recomputes the softmax from the saved per-row logsumexp
// instead of storing the R*H*N*N probabilities (the pages' memory-efficient
// kernel runs in the forward and the backward pass: gist.science MegaFold
// technical summary, Methodik section 1 "EvoFlash-3D").  With dS = P * (dP - D),
// D[j] = sum_c dO[j,c] O[j,c], the gradients are
//   dV = P^T dO,  dK = dS^T Q / sqrt(d),  dQ = dS K / sqrt(d),
//   dBias[h,j,k] = sum over rows r of dS[r,h,j,k].
//
// Three kernels each own complete outputs, so nothing is accumulated with
// atomics and every sum has a fixed order:
//  * dkdv : workgroup = 128 keys (4 waves x 32) of one (row, head); walks the
//           queries in steps of 64.  Tiles are S = Q K^T (queries x keys): each
//           lane holds one key, so P and dS in registers are directly the B
//           operands of dV^T = dO^T P and dK^T = Q^T dS.
//  * dq   : workgroup = 128 queries of one (row, head); walks the keys in steps
//           of 64 with the forward's transposed tiles S^T = K Q^T, so dS^T in
//           registers is the B operand of dQ^T = K^T dS^T.
//  * dbias: workgroup = a 64 x 128 (query x key) tile of one head; walks a group
//           of rows in increasing order and sums dS in registers.  Row groups
//           give partial sums that a last kernel adds in increasing group order.
// Scaled bias (sqrt(d) * bias, fp32) initialises every S accumulator and -D
// initialises every dP accumulator, so neither costs vector ALU work.

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;

// Per-query statistics of a step of queries: -lse in log2 units (-inf gives
// P = 0 for padded queries and for rows whose keys are all masked) and -D.
struct StatStage {
  float nl, nd;
  __device__ __forceinline__ void load(const Problem& p, const BwdArgs& a, int r, int h, int q0) {
    nl = -INFINITY;
    nd = 0.f;
    const int j = q0 + static_cast<int>(threadIdx.x);
    if (threadIdx.x < kStep && j < p.N) {
      const int64_t id = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
      const float l = a.lse[id];
      if (l != -INFINITY) nl = -l * kLog2e;
      nd = -a.delta[id];
    }
  }
  __device__ __forceinline__ void store(float* nlse, float* ndel) const {
    if (threadIdx.x < kStep) {
      nlse[threadIdx.x] = nl;
      ndel[threadIdx.x] = nd;
    }
  }
};

// ------------------------------------------------------------------ dK, dV
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(Problem p, BwdArgs a, const float* __restrict__ bias_t,
                                                               int np) {
  using S = Shape<D>;
  __shared__ __align__(16) uint16_t q_rows[2][kStep * S::ROW];
  __shared__ __align__(16) uint16_t q_trans[2][S::DB * 32 * S::TROW];
  __shared__ __align__(16) uint16_t do_rows[2][kStep * S::ROW];
  __shared__ __align__(16) uint16_t do_trans[2][S::DB * 32 * S::TROW];
  __shared__ __align__(16) float nlse_lds[2][kStep];
  __shared__ __align__(16) float ndel_lds[2][kStep];

  const int nkb = (p.N + 127) / 128;
  int blk = blockIdx.x;
  const int kb = blk % nkb;
  blk /= nkb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int key = kb * 128 + wave * 32 + col;  // < np

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;

  u32x4 kreg[S::KS], vreg[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) {
    kreg[ks] = global_operand<D>(p, k, r, key, h, ks, half);
    vreg[ks] = global_operand<D>(p, v, r, key, h, ks, half);
  }
  const bool valid = key < p.N;
  const float mk = (a.mask && valid) ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
  const bool wave_live = __ballot(valid && mk != -INFINITY) != 0;
  const bool any_mask = __ballot(valid && mk != 0.f) != 0;
  const float mk_s = sd * mk;

  f32x16 dv_acc[S::DB], dk_acc[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dv_acc[db][i] = dk_acc[db][i] = 0.f;

  const float* brow = bias_t + (static_cast<int64_t>(h) * np + key) * np;  // bias^T row of this key

  const int64_t rh = row_head_offset(p, r, h);
  const int64_t pstep = pos_step(p);
  const uint16_t* qbase = q + rh;
  const uint16_t* dobase = dout + rh;
  Stage<D> qst, dost;
  qst.init(p);
  dost.init(p);
  StatStage stst;
  f32x16 bnext[2];
  qst.load(qbase, 0, p.N);
  dost.load(dobase, 0, p.N);
  stst.load(p, a, r, h, 0);
  if (wave_live) {
    bnext[0] = load_acc_rows(brow, half);
    bnext[1] = load_acc_rows(brow + 32, half);
  }

  int buf = 0;
  for (int q0 = 0; q0 < p.N; q0 += kStep) {
    qst.store(q_rows[buf], q_trans[buf], S::ROW, q0, p.N);
    dost.store(do_rows[buf], do_trans[buf], S::ROW, q0, p.N);
    stst.store(nlse_lds[buf], ndel_lds[buf]);
    lds_barrier();
    const int cb = buf;
    buf ^= 1;
    // S = Q K^T + sqrt(d) (bias + mask): rows = queries q0 + 32 qt + ..., lane = key.
    f32x16 s[2];
    if (wave_live) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x16 c = bnext[qt];
        if (any_mask) c += mk_s;
        s[qt] = mma(rows_operand<D>(q_rows[cb], 32 * qt, 0, col, half), kreg[0], c);
#pragma unroll
        for (int ks = 1; ks < S::KS; ++ks) s[qt] = mma(rows_operand<D>(q_rows[cb], 32 * qt, ks, col, half), kreg[ks], s[qt]);
      }
    }
    const int q1 = q0 + kStep;
    if (q1 < p.N) {
      qst.load(qbase + q1 * pstep, q1, p.N);
      dost.load(dobase + q1 * pstep, q1, p.N);
      stst.load(p, a, r, h, q1);
      if (wave_live) {
        bnext[0] = load_acc_rows(brow + q1, half);
        bnext[1] = load_acc_rows(brow + q1 + 32, half);
      }
    }
    if (!wave_live) continue;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const f32x16 nl = load_acc_rows(&nlse_lds[cb][32 * qt], half);
      // dP - D = dO V^T - D.
      f32x16 dp = load_acc_rows(&ndel_lds[cb][32 * qt], half);
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) dp = mma(rows_operand<D>(do_rows[cb], 32 * qt, ks, col, half), vreg[ks], dp);
      u32x4 pb[2], dsb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[8], dsv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = fast_exp2(__builtin_fmaf(s[qt][8 * t + i], c1, nl[8 * t + i]));
          dsv[i] = pv[i] * dp[8 * t + i];
        }
        pb[t] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                      pack_bf16(pv[6], pv[7])};
        dsb[t] = u32x4{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                       pack_bf16(dsv[6], dsv[7])};
      }
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          dv_acc[db] = mma(trans_operand<D>(do_trans[cb], db, 32 * qt, t, col, half), pb[t], dv_acc[db]);
          dk_acc[db] = mma(trans_operand<D>(q_trans[cb], db, 32 * qt, t, col, half), dsb[t], dk_acc[db]);
        }
      }
    }
  }
  if (!valid) return;
  const int64_t off = elem_offset(p, r, key, h);
  store_dT<D>(static_cast<uint16_t*>(a.dv) + off, dv_acc, 1.f, half);
  store_dT<D>(static_cast<uint16_t*>(a.dk) + off, dk_acc, 1.f / sd, half);
}

// ------------------------------------------------------------------ dQ
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(Problem p, BwdArgs a, const float* __restrict__ bias_f,
                                                             int np) {
  using S = Shape<D>;
  __shared__ __align__(16) uint16_t k_rows[2][kStep * S::ROW];
  __shared__ __align__(16) uint16_t k_trans[2][S::DB * 32 * S::TROW];
  __shared__ __align__(16) uint16_t v_rows[2][kStep * S::ROW];
  __shared__ __align__(16) float m_lds[2][kStep];
  __shared__ __align__(16) float ndel4[4][32][4];  // -D of each wave's queries, replicated 4x

  const int nqb = (p.N + 127) / 128;
  int blk = blockIdx.x;
  const int qb = blk % nqb;
  blk /= nqb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int j0 = qb * 128 + wave * 32;
  const int j = j0 + col;  // < np
  const bool wave_active = j0 < p.N;

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;

  u32x4 qreg[S::KS], doreg[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) {
    qreg[ks] = global_operand<D>(p, q, r, j, h, ks, half);
    doreg[ks] = global_operand<D>(p, dout, r, j, h, ks, half);
  }
  float nl = -INFINITY, nd = 0.f;
  if (j < p.N) {
    const int64_t id = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
    const float l = a.lse[id];
    if (l != -INFINITY) nl = -l * kLog2e;
    nd = -a.delta[id];
  }
  if (half == 0) *reinterpret_cast<f32x4*>(&ndel4[wave][col][0]) = f32x4{nd, nd, nd, nd};
  const bool row_live = wave_active && __ballot(nl != -INFINITY) != 0;

  f32x16 dq_acc[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_acc[db][i] = 0.f;

  const float* mrow = a.mask ? a.mask + static_cast<int64_t>(r) * p.N : nullptr;

  const int64_t rh = row_head_offset(p, r, h);
  const int64_t pstep = pos_step(p);
  const uint16_t* kbase = k + rh;
  const uint16_t* vbase = v + rh;
  const float* bhead = bias_f + static_cast<int64_t>(h) * np * np;
  const uint32_t boff = static_cast<uint32_t>(j * np);
  Stage<D> kst, vst;
  kst.init(p);
  vst.init(p);
  f32x16 bnext[2];
  float mnext = 0.f;
  kst.load(kbase, 0, p.N);
  vst.load(vbase, 0, p.N);
  if (mrow) mnext = mrow[min(lane, p.N - 1)];
  if (row_live) {
    bnext[0] = load_acc_rows(bhead + boff, half);
    bnext[1] = load_acc_rows(bhead + boff + 32, half);
  }

  int buf = 0;
  for (int k0 = 0; k0 < p.N; k0 += kStep) {
    const bool kvalid = k0 + lane < p.N;
    const float mv = kvalid ? mnext : 0.f;
    const bool live = __ballot(kvalid && mv != -INFINITY) != 0;
    const bool any_mask = __ballot(kvalid && mv != 0.f) != 0;
    const bool compute = live && row_live;
    const int cb = buf;
    if (live) {
      kst.store(k_rows[buf], k_trans[buf], S::ROW, k0, p.N);
      vst.store(v_rows[buf], nullptr, S::ROW, k0, p.N);
      if (any_mask && tid < kStep) m_lds[buf][tid] = kvalid ? sd * mv : -INFINITY;
      lds_barrier();
      buf ^= 1;
    }
    // S^T = K Q^T + sqrt(d) (bias + mask): rows = keys k0 + 32 mb + ..., lane = query.
    f32x16 s[2];
    if (compute) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 c = bnext[mb];
        if (any_mask) c += load_acc_rows(&m_lds[cb][32 * mb], half);
        s[mb] = mma(rows_operand<D>(k_rows[cb], 32 * mb, 0, col, half), qreg[0], c);
#pragma unroll
        for (int ks = 1; ks < S::KS; ++ks) s[mb] = mma(rows_operand<D>(k_rows[cb], 32 * mb, ks, col, half), qreg[ks], s[mb]);
      }
    }
    const int k1 = k0 + kStep;
    if (k1 < p.N) {
      kst.load(kbase + k1 * pstep, k1, p.N);
      vst.load(vbase + k1 * pstep, k1, p.N);
      if (mrow) mnext = mrow[min(k1 + lane, p.N - 1)];
      if (row_live) {
        bnext[0] = load_acc_rows(bhead + k1 + boff, half);
        bnext[1] = load_acc_rows(bhead + k1 + boff + 32, half);
      }
    }
    if (!compute) continue;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // dP^T - D = V dO^T - D; the accumulator starts at -D of the lane's query.
      f32x16 dp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&ndel4[wave][col][0]);
        dp[4 * g + 0] = x[0];
        dp[4 * g + 1] = x[1];
        dp[4 * g + 2] = x[2];
        dp[4 * g + 3] = x[3];
      }
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) dp = mma(rows_operand<D>(v_rows[cb], 32 * mb, ks, col, half), doreg[ks], dp);
      u32x4 dsb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float dsv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) dsv[i] = fast_exp2(__builtin_fmaf(s[mb][8 * t + i], c1, nl)) * dp[8 * t + i];
        dsb[t] = u32x4{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                       pack_bf16(dsv[6], dsv[7])};
      }
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          dq_acc[db] = mma(trans_operand<D>(k_trans[cb], db, 32 * mb, t, col, half), dsb[t], dq_acc[db]);
    }
  }
  if (!wave_active || j >= p.N) return;
  store_dT<D>(static_cast<uint16_t*>(a.dq) + elem_offset(p, r, j, h), dq_acc, 1.f / sd, half);
}

// dbias[i] = sum over groups g = 0, 1, ... of part[g][i], in increasing g.
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float* __restrict__ part, int groups, int64_t n,
                                                           float* __restrict__ dbias) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = part[i];
    for (int g = 1; g < groups; ++g) s += part[static_cast<int64_t>(g) * n + i];
    dbias[i] = s;
  }
}

// Per-row terms of the backward, one thread per (r, j, h) in memory order (so a
// wave reads contiguous 2*d-byte pieces of O and dO):
//   delta[r,h,j] = sum_c dout[r,j,h,c] o[r,j,h,c]
//   qaug[r,h,j]  = the query-side split operands of -sqrt(d) lse and -delta
//   kaug[r,j]    = the key-side split operands of sqrt(d) mask (threads with h = 0)
// (layouts of the operands: pipe_common.h).
template <int D>
__global__ __launch_bounds__(256) void bwd_rowterms_kernel(Problem p, BwdArgs a) {
  using namespace pipe;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(p.R) * p.H * p.N;
  if (idx >= total) return;
  const int h = static_cast<int>(idx % p.H);
  const int64_t pr = idx / p.H;  // (r, j) or (j, r) in memory order
  const int r = static_cast<int>(p.transpose ? pr % p.R : pr / p.N);
  const int j = static_cast<int>(p.transpose ? pr / p.R : pr % p.N);
  const int64_t off = idx * D;
  const u32x4* o = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.o) + off);
  const u32x4* d = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dout) + off);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 x = o[c], y = d[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += __uint_as_float(x[i] << 16) * __uint_as_float(y[i] << 16);
      s += __uint_as_float(x[i] & 0xffff0000u) * __uint_as_float(y[i] & 0xffff0000u);
    }
  }
  const int64_t rhj = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
  a.delta[rhj] = s;
  const float sd = sqrtf(static_cast<float>(D));
  const Split3 na = split3(-lse_term(a.lse[rhj], sd, true));
  const Split3 nd = split3(-s);
  reinterpret_cast<u32x4*>(a.qaug)[rhj] =
      u32x4{na.hi | (na.mid << 16), na.lo | (kBf16One << 16), nd.hi | (nd.mid << 16), nd.lo};
  if (h == 0) {
    const float m = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + j] : 0.f;
    const Split3 sm = split3(fmaxf(sd * m, -kHuge));
    reinterpret_cast<u32x4*>(a.kaug)[static_cast<int64_t>(r) * p.N + j] =
        u32x4{kBf16One | (kBf16One << 16), kBf16One | (sm.hi << 16), sm.mid | (sm.lo << 16), 0u};
  }
}

template <int D>
hipError_t bwd_mfma_dispatch(const Problem& p, const BwdArgs& a, float* bias_f, float* bias_t, float* bias_k, int np,
                             float* dbias_part, int groups, hipStream_t s) {
  hipError_t e;
  {
    const int64_t rows_total = static_cast<int64_t>(p.R) * p.H * p.N;
    KernelTimer timer("bwd_rowterms", s);
    hipLaunchKernelGGL((bwd_rowterms_kernel<D>), dim3(static_cast<unsigned>((rows_total + 255) / 256)), dim3(256), 0,
                       s, p, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_bias_prep(p, a.bias, bias_t, np, 1, s)) != hipSuccess) return e;
  if ((e = launch_bias_prep(p, a.bias, bias_f, np, 0, s)) != hipSuccess) return e;
  if ((e = launch_bias_tiles(p, a.bias, bias_k, 1, s)) != hipSuccess) return e;
  if ((e = launch_dkdv_pipe(p, a, bias_k, s)) != hipSuccess) return e;
  {
    const int64_t blocks = static_cast<int64_t>((p.N + 127) / 128) * p.H * p.R;
    KernelTimer timer("bwd_dq_mfma", s);
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, p, a, bias_f,
                       np);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.dbias) {
    float* target = groups == 1 ? a.dbias : dbias_part;
    if ((e = launch_dbias_pipe(p, a, bias_k, groups, target, s)) != hipSuccess) return e;
    if (groups > 1) {
      const int64_t n = static_cast<int64_t>(p.H) * p.N * p.N;
      const int rb = static_cast<int>(std::min<int64_t>((n + 255) / 256, 4096));
      KernelTimer timer("bwd_dbias_reduce", s);
      hipLaunchKernelGGL(dbias_reduce_kernel, dim3(rb), dim3(256), 0, s, dbias_part, groups, n, a.dbias);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Workspace: delta [R,H,N] | qaug [R,H,N] x 16 B | kaug [R,N] x 16 B |
// bias_f, bias_t [H,np,np] | tiled bias (key lanes) | dbias partials [G,H,N,N].
size_t bwd_mfma_workspace_bytes(const Problem& p) {
  const size_t np = static_cast<size_t>(bias_pad(p.N));
  const int groups = dbias_pipe_groups(p);
  const size_t delta = align_up(static_cast<size_t>(p.R) * p.H * p.N * sizeof(float)) +
                       align_up(static_cast<size_t>(p.R) * p.H * p.N * 16) + align_up(static_cast<size_t>(p.R) * p.N * 16);
  const size_t bias = align_up(static_cast<size_t>(p.H) * np * np * sizeof(float));
  const size_t tiled = align_up(tiled_bias_bytes(p));
  const size_t part = groups > 1 ? align_up(static_cast<size_t>(groups) * p.H * p.N * p.N * sizeof(float)) : 0;
  return delta + 2 * bias + tiled + part;
}

hipError_t launch_bwd_mfma(const Problem& p, const BwdArgs& args, void* ws, hipStream_t s) {
  const size_t np = static_cast<size_t>(bias_pad(p.N));
  const int groups = dbias_pipe_groups(p);
  char* base = static_cast<char*>(ws);
  BwdArgs a = args;
  a.delta = reinterpret_cast<float*>(base);
  base += align_up(static_cast<size_t>(p.R) * p.H * p.N * sizeof(float));
  a.qaug = base;
  base += align_up(static_cast<size_t>(p.R) * p.H * p.N * 16);
  a.kaug = base;
  base += align_up(static_cast<size_t>(p.R) * p.N * 16);
  float* bias_f = reinterpret_cast<float*>(base);
  base += align_up(static_cast<size_t>(p.H) * np * np * sizeof(float));
  float* bias_t = reinterpret_cast<float*>(base);
  base += align_up(static_cast<size_t>(p.H) * np * np * sizeof(float));
  float* bias_k = reinterpret_cast<float*>(base);
  base += align_up(tiled_bias_bytes(p));
  float* part = reinterpret_cast<float*>(base);
  switch (p.D) {
    case 8: return bwd_mfma_dispatch<8>(p, a, bias_f, bias_t, bias_k, static_cast<int>(np), part, groups, s);
    case 16: return bwd_mfma_dispatch<16>(p, a, bias_f, bias_t, bias_k, static_cast<int>(np), part, groups, s);
    case 32: return bwd_mfma_dispatch<32>(p, a, bias_f, bias_t, bias_k, static_cast<int>(np), part, groups, s);
    case 64: return bwd_mfma_dispatch<64>(p, a, bias_f, bias_t, bias_k, static_cast<int>(np), part, groups, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evo
