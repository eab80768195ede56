// Backward of pair-biased 3D attention on the bf16 MFMA path (gfx950): the
// per-row pre-pass, the launch sequence and the workspace layout.
//
// The backward recomputes the softmax from the saved per-row logsumexp instead
// of storing the R*H*N*N probabilities (the pages' memory-efficient kernel runs
// in the forward and the backward pass: gist.science MegaFold technical
// summary, Methodik section 1 "EvoFlash-3D").  With dS = P * (dP - D),
// D[j] = sum_c dO[j,c] O[j,c], the gradients are
//   dV = P^T dO,  dK = dS^T Q / sqrt(d),  dQ = dS K / sqrt(d),
//   dBias[h,j,k] = sum over rows r of dS[r,h,j,k].
// Every kernel owns complete outputs, so nothing is accumulated with atomics
// and every sum has a fixed order:
//  * fused (kernels_bwd_fused.hip), head_dim <= 32 and N <= 384: a workgroup owns
//    one attention row of one head and forms its dQ, dK and dV from one pass over
//    the score tiles;
//  * otherwise dq (kernels_bwd_dq.hip), where a workgroup owns queries and walks
//    the keys, and dkdv (kernels_bwd_dkdv.hip), where it owns keys and walks the
//    queries;
//  * dbias (kernels_bwd_dbias.hip): a workgroup owns a (query, key) tile of a
//    head and walks a fixed group of rows; the groups' partial sums are added in
//    increasing group order by the fused kernel once its rows are done (the dbias
//    pass then runs before it) or by a last pass after dq and dkdv.
// Per-row terms (lse, D, the key mask) enter the MFMA accumulators as exact
// split-bf16 operands prepared once by bwd_rowterms_kernel.

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

using namespace mfma;

// dbias[i] = sum over groups g = 0, 1, ... of part[g][i], in increasing g (a
// grid-stride pass of pipe::dbias_reduce_range).
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float* __restrict__ part, int groups, int64_t n,
                                                           float* __restrict__ dbias) {
  dbias_reduce_range(part, groups, n, dbias, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                     static_cast<int64_t>(gridDim.x) * blockDim.x);
}

// Per-row terms of the backward, D = sum_c dout[r,j,h,c] o[r,j,h,c]:
//   qops[r,h,j]  = the complete query-side operands of the S and dP steps
//                  (-sqrt(d) lse and -D, split; dbias and the fused kernel)
//   qaug[r,h,j]  = the same in the packed form of the dq and dkdv kernels (only
//                  when those run)
//   kaug[r,j]    = the key-side split operands of sqrt(d) mask (h = 0)
// (layouts of the operands: pipe_common.h).  One thread per (r, j, h):
//  * [R, N, H, d] layout with H in {1, 2, 4, 8} ("staged"): a workgroup takes
//    256 / H consecutive queries of one row with all heads, so it reads one
//    contiguous piece of O and dO; the operands go through LDS and leave as
//    contiguous runs per head;
//  * otherwise the order (r, h, j), j fastest (a lane reads the 2 d contiguous
//    bytes of its query, and operand writes are contiguous in j).
// The same launch also forms the sqrt(d) * bias tiles the later kernels read:
// blocks 0 .. tiles - 1 each form one tile (pipe::bias_tile), so that this small
// pass overlaps the row terms instead of taking a launch of its own.
template <int D>
__global__ __launch_bounds__(256) void bwd_rowterms_kernel(Problem p, BwdArgs a, float* __restrict__ bias_q,
                                                           float* __restrict__ bias_k, int nt, int tiles,
                                                           bool staged) {
  using namespace pipe;
  if (static_cast<int>(blockIdx.x) < tiles) {
    bias_tile(p, static_cast<const uint16_t*>(a.bias), bias_q, bias_k, nt, blockIdx.x);
    return;
  }
  const int64_t blk = static_cast<int64_t>(blockIdx.x) - tiles;
  const int t = threadIdx.x;
  int r, j, h, jq = 0, j0 = 0;  // jq: queries per workgroup (staged)
  bool valid;
  if (staged) {
    jq = 256 / p.H;
    const int chunks = (p.N + jq - 1) / jq;
    r = static_cast<int>(blk / chunks);
    j0 = static_cast<int>(blk % chunks) * jq;
    j = j0 + t / p.H;
    h = t % p.H;
    valid = j < p.N;
  } else {
    const int64_t idx = blk * 256 + t;
    valid = idx < static_cast<int64_t>(p.R) * p.H * p.N;
    j = static_cast<int>(idx % p.N);
    const int64_t rh_idx = idx / p.N;
    h = static_cast<int>(rh_idx % p.H);
    r = static_cast<int>(rh_idx / p.H);
  }
  const float sd = sqrtf(static_cast<float>(D));
  const int np = qops_queries(p.N);
  u32x4 sq{}, dq{}, qa{};
  if (valid) {
    const int64_t off = elem_offset(p, r, j, h);
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
    const Split3 na = split3(-lse_term(a.lse[rhj], sd, true));
    const Split3 nd = split3(-s);
    qa = u32x4{na.hi | (na.mid << 16), na.lo | (kBf16One << 16), nd.hi | (nd.mid << 16), nd.lo};
    sq = u32x4{na.hi | (na.mid << 16), na.lo | (kBf16One << 16), kBf16One | (kBf16One << 16), 0u};
    dq = u32x4{nd.hi | (nd.mid << 16), nd.lo, 0u, 0u};
    u32x4* qo = reinterpret_cast<u32x4*>(a.qops) + 2 * (static_cast<int64_t>(r) * p.H + h) * np;
    if (!staged) {
      if (a.qaug) reinterpret_cast<u32x4*>(a.qaug)[rhj] = qa;
      qo[(j >> 5) * 64 + (j & 31)] = sq;
      qo[(j >> 5) * 64 + 32 + (j & 31)] = dq;
    }
    // The padding queries N .. Np - 1 of the row get the dead-query side (every
    // probability 0) from the thread of query N - 1.
    if (j == p.N - 1)
      for (int jj = p.N; jj < np; ++jj) {
        qo[(jj >> 5) * 64 + (jj & 31)] = dead_query_aug();
        qo[(jj >> 5) * 64 + 32 + (jj & 31)] = u32x4{0u, 0u, 0u, 0u};
      }
    if (h == 0) {
      const float m = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + j] : 0.f;
      const Split3 sm = split3(fmaxf(sd * m, -kHuge));
      reinterpret_cast<u32x4*>(a.kaug)[static_cast<int64_t>(r) * p.N + j] =
          u32x4{kBf16One | (kBf16One << 16), kBf16One | (sm.hi << 16), sm.mid | (sm.lo << 16), 0u};
    }
  }
  if (!staged) return;
  // Staged: through LDS, [h][query] per operand, then out as contiguous runs.
  __shared__ u32x4 st_s[256], st_d[256], st_q[256];
  const int slot = h * jq + (j - j0);
  st_s[slot] = sq;
  st_d[slot] = dq;
  st_q[slot] = qa;
  __syncthreads();
  // qops: per head the jq queries are jq / 32 whole blocks, 2 jq consecutive entries.
#pragma unroll
  for (int e = t; e < 512; e += 256) {
    const int hh = e / (2 * jq), w = e % (2 * jq);
    const int jl = (w >> 6) * 32 + (w & 31);
    if (j0 + jl < p.N) {
      u32x4* qo = reinterpret_cast<u32x4*>(a.qops) + 2 * (static_cast<int64_t>(r) * p.H + hh) * np;
      qo[(j0 >> 5) * 64 + w] = (w & 32) ? st_d[hh * jq + jl] : st_s[hh * jq + jl];
    }
  }
  if (a.qaug) {
    const int hh = t / jq, jl = t % jq;
    if (j0 + jl < p.N)
      reinterpret_cast<u32x4*>(a.qaug)[(static_cast<int64_t>(r) * p.H + hh) * p.N + j0 + jl] = st_q[hh * jq + jl];
  }
}

}  // namespace

namespace {

template <int D>
hipError_t bwd_mfma_dispatch(const Problem& p, const BwdArgs& a, float* bias_q, float* bias_k, float* dbias_part,
                             int groups, hipStream_t s) {
  hipError_t e;
  const bool fused = bwd_fused_supported(p);
  {
    // Row terms and the bias tiles: key-lane tiles always, query-lane tiles for
    // the dq kernel.
    const int64_t rows_total = static_cast<int64_t>(p.R) * p.H * p.N;
    const int nt = bias_tiles(p.N);
    const int tiles = p.H * nt * nt;
    const bool staged = !p.transpose && (p.H == 1 || p.H == 2 || p.H == 4 || p.H == 8);
    const int64_t row_blocks = staged ? static_cast<int64_t>(p.R) * ((p.N + 256 / p.H - 1) / (256 / p.H))
                                      : (rows_total + 255) / 256;
    KernelTimer timer("bwd_prep", s);
    hipLaunchKernelGGL((bwd_rowterms_kernel<D>), dim3(static_cast<unsigned>(tiles + row_blocks)), dim3(256), 0, s, p,
                       a, fused ? nullptr : bias_q, bias_k, nt, tiles, staged);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // The fused pass adds the dBias partials up itself after its rows, so there the
  // dBias pass runs first; otherwise a separate reduce pass follows it.
  const bool partials = a.dbias && groups > 1;
  if (fused) {
    if (a.dbias && (e = launch_dbias_pipe(p, a, bias_k, groups, partials ? dbias_part : a.dbias, s)) != hipSuccess)
      return e;
    return launch_bwd_fused(p, a, bias_k, partials ? dbias_part : nullptr, groups, s);
  }
  if ((e = launch_dq_pipe(p, a, bias_q, s)) != hipSuccess) return e;
  if ((e = launch_dkdv_pipe(p, a, bias_k, s)) != hipSuccess) return e;
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

struct BwdLayout {
  size_t qaug, kaug, bias, part, qops, total;
};
BwdLayout bwd_layout(const Problem& p) {
  BwdLayout l;
  const int groups = dbias_pipe_groups(p);
  l.qaug = bwd_fused_supported(p) ? 0 : align_up(static_cast<size_t>(p.R) * p.H * p.N * 16);
  l.kaug = align_up(static_cast<size_t>(p.R) * p.N * 16);
  l.bias = align_up(tiled_bias_bytes(p));
  l.part = groups > 1 ? align_up(static_cast<size_t>(groups) * p.H * p.N * p.N * sizeof(float)) : 0;
  l.qops = align_up(static_cast<size_t>(p.R) * p.H * qops_queries(p.N) * 32);
  l.total = l.qaug + l.kaug + 2 * l.bias + l.part + l.qops;
  return l;
}

}  // namespace

// Workspace: qaug [R,H,N] x 16 B (when the dq and dkdv kernels run) | kaug [R,N] x 16 B |
// tiled bias, query lanes | tiled bias, key lanes | dbias partials [G,H,N,N] fp32 |
// query operands qops [R,H,Np] x 32 B (Np = qops_queries(N)).
size_t bwd_mfma_workspace_bytes(const Problem& p) { return bwd_layout(p).total; }

hipError_t launch_bwd_mfma(const Problem& p, const BwdArgs& args, void* ws, hipStream_t s) {
  const BwdLayout l = bwd_layout(p);
  const int groups = dbias_pipe_groups(p);
  char* base = static_cast<char*>(ws);
  BwdArgs a = args;
  a.delta = nullptr;  // D lives in qops (and qaug) on this path
  a.qaug = l.qaug ? base : nullptr;
  base += l.qaug;
  a.kaug = base;
  base += l.kaug;
  float* bias_q = reinterpret_cast<float*>(base);
  base += l.bias;
  float* bias_k = reinterpret_cast<float*>(base);
  base += l.bias;
  float* part = reinterpret_cast<float*>(base);
  base += l.part;
  a.qops = base;
  switch (p.D) {
    case 8: return bwd_mfma_dispatch<8>(p, a, bias_q, bias_k, part, groups, s);
    case 16: return bwd_mfma_dispatch<16>(p, a, bias_q, bias_k, part, groups, s);
    case 32: return bwd_mfma_dispatch<32>(p, a, bias_q, bias_k, part, groups, s);
    case 64: return bwd_mfma_dispatch<64>(p, a, bias_q, bias_k, part, groups, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evo
