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

constexpr int kFwdThreads = 256;
constexpr int kFwdQueries = 128;  // per workgroup
constexpr int kFwdKeys = 64;      // per step

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
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_mfma_kernel(Problem p, FwdArgs a,
                                                                   const float* __restrict__ bias_s, int nqp,
                                                                   int nkp) {
  constexpr int KS = D >= 16 ? D / 16 : 1;  // 16-deep steps of the Q.K contraction
  constexpr int DB = D >= 32 ? D / 32 : 1;  // 32-row blocks of O^T
  constexpr int KROW = KS * 16 + 8;         // bf16 per staged K row (8 padding)
  constexpr int VROW = kFwdKeys + 8;        // bf16 per staged V^T row (8 padding)
  constexpr int CHUNKS = D / 8;             // 16-byte chunks per key row
  __shared__ __align__(16) uint16_t k_lds[kFwdKeys * KROW];
  __shared__ __align__(16) uint16_t vt_lds[DB * 32 * VROW];
  __shared__ __align__(16) float m_lds[kFwdKeys];

  const int nqb = (p.N + kFwdQueries - 1) / kFwdQueries;
  int blk = blockIdx.x;
  const int qb = blk % nqb;
  blk /= nqb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int j0 = qb * kFwdQueries + wave * 32;
  const int j = j0 + col;  // this lane's query
  const bool wave_active = j0 < p.N;

  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const float sd = sqrtf(static_cast<float>(D));
  const float c1 = kLog2e / sd;

  // Q as the B operand of S^T = K Q^T: query = col, d = 16 ks + 8 half + i.
  u32x4 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = ks * 16 + 8 * half;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (j < p.N && d0 < D) val = *reinterpret_cast<const u32x4*>(q + elem_offset(p, r, j, h) + d0);
    qreg[ks] = val;
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY;  // running max of the scaled (log2) logits of this query
  float l_run = 0.f;        // this lane's share of the running sum

  const float* brow = bias_s + (static_cast<int64_t>(h) * nqp + j) * nkp;
  const float* mrow = a.mask ? a.mask + static_cast<int64_t>(r) * p.N : nullptr;

  for (int k0 = 0; k0 < p.N; k0 += kFwdKeys) {
    // Classify the block by its mask (same answer in every wave of the workgroup).
    const int key = k0 + lane;
    const bool valid = key < p.N;
    const float mv = (mrow && valid) ? mrow[key] : 0.f;
    const uint64_t live = __ballot(valid && mv != -INFINITY);
    if (live == 0) continue;
    const bool any_mask = __ballot(valid && mv != 0.f) != 0;

    __syncthreads();  // the previous block's LDS readers are done
    for (int c = tid; c < kFwdKeys * CHUNKS; c += kFwdThreads) {
      const int kr = c / CHUNKS;
      const int ch = c % CHUNKS;
      const int kk = k0 + kr;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (kk < p.N) {
        const int64_t off = elem_offset(p, r, kk, h) + ch * 8;
        kv = *reinterpret_cast<const u32x4*>(k + off);
        vv = *reinterpret_cast<const u32x4*>(v + off);
      }
      *reinterpret_cast<u32x4*>(&k_lds[kr * KROW + ch * 8]) = kv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vt_lds[(ch * 8 + 2 * i) * VROW + kr] = static_cast<uint16_t>(vv[i] & 0xffffu);
        vt_lds[(ch * 8 + 2 * i + 1) * VROW + kr] = static_cast<uint16_t>(vv[i] >> 16);
      }
    }
    if (any_mask && tid < kFwdKeys) m_lds[tid] = valid ? sd * mv : -INFINITY;
    __syncthreads();
    if (!wave_active) continue;

    // S^T tiles for keys k0 + [0,32) and k0 + [32,64).
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(brow + k0 + mb * 32 + 8 * g + 4 * half);
        s[mb][4 * g + 0] = b4[0];
        s[mb][4 * g + 1] = b4[1];
        s[mb][4 * g + 2] = b4[2];
        s[mb][4 * g + 3] = b4[3];
      }
      if (any_mask) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 m4 = *reinterpret_cast<const f32x4*>(&m_lds[mb * 32 + 8 * g + 4 * half]);
          s[mb][4 * g + 0] += m4[0];
          s[mb][4 * g + 1] += m4[1];
          s[mb][4 * g + 2] += m4[2];
          s[mb][4 * g + 3] += m4[3];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 kop = {0u, 0u, 0u, 0u};
        if (D >= 16 || half == 0) kop = *reinterpret_cast<const u32x4*>(&k_lds[(mb * 32 + col) * KROW + ks * 16 + 8 * half]);
        s[mb] = mma(kop, qreg[ks], s[mb]);
      }
    }

    // Online softmax over this block's keys (exp2 domain).
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c1);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    u32x4 pb[2][2];  // P^T packed to bf16: [key tile][16-key half]
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = fast_exp2(__builtin_fmaf(s[mb][8 * t + i], c1, -m_new));
          l_run += pv[i];
        }
        pb[mb][t] = u32x4{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                          pack_bf16(pv[6], pv[7])};
      }
    }

    // O^T += V^T P^T over the 64 keys (four 16-deep steps).
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vrow = &vt_lds[(db * 32 + col) * VROW];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int kb0 = mb * 32 + 16 * t + 4 * half;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kb0);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + kb0 + 8);
          oacc[db] = mma(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb[mb][t], oacc[db]);
        }
      }
    }
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  if (j >= p.N) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* o = static_cast<uint16_t*>(a.o) + elem_offset(p, r, j, h);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * half;
      if (d < D) {
        const u32x2 w = {pack_bf16(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                         pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(o + d) = w;
      }
    }
  }
  if (a.lse && half == 0)
    a.lse[(static_cast<int64_t>(r) * p.H + h) * p.N + j] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t fwd_mfma_dispatch(const Problem& p, const FwdArgs& a, float* bias_s, int np, hipStream_t s) {
  hipError_t e = launch_bias_prep(p, a.bias, bias_s, np, 0, s);
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>((p.N + kFwdQueries - 1) / kFwdQueries) * p.H * p.R;
  KernelTimer timer("fwd_mfma", s);
  hipLaunchKernelGGL((fwd_mfma_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(kFwdThreads), 0, s, p, a,
                     bias_s, np, np);
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
