// Fused layer norm + projections of a token tensor into the attention's inputs
// (MegaFold, gist.science technical summary, Methodik section 3 "EvoFusion":
// layer norm and the linear projections after it run as one operator, so the
// normalised N x N tensor never goes to HBM between the two).
//
// For every token t of x [A, B, C]:  y = (x - mean) * rstd * gamma + beta with
// the biased variance and rstd = 1/sqrt(var + eps); then
//   q/k/v[t][h*D + e] = sum_c y[c] w_qkv[o][c]   (o = which*H*D + h*D + e)
//   bias[h][a][b]     = sum_c y[c] w_bias[h][c]  (token (a, b), or (b, a) when
//                                                 bias_transpose is set)
// q, k, v keep x's token order, which is the attention's kernel frame for the
// starting node and its transposed frame for the ending node.
//
// bf16 with C in {32, 64, 128}: one MFMA kernel.  A workgroup copies all
// projection weights into LDS once and its waves then stream 32-token tiles:
// x arrives straight in the MFMA operand layout, layer-norm statistics come from
// registers (each token's channels sit on two lanes), the normalised tile is
// rounded to bf16 in registers and multiplied by every weight tile.  Per token
// HBM sees C reads and n_out writes; nothing in between.
// Other shapes and fp32: a plain vector kernel with the same semantics.

#include <hip/hip_runtime.h>

#include "evoattn_internal.h"
#include "mfma_common.h"
#include "pipe_common.h"
#include "proj_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace proj;

constexpr int kProjWaves = 8;
constexpr int kProjThreads = 64 * kProjWaves;

// ---------------------------------------------------------------- bf16 MFMA kernel

// LDS: gamma[C], beta[C] (fp32), then weight rows [n_tiles*32][C] bf16 with a
// pitch of 2C + 16 bytes, which spreads the 32 rows a ds_read_b128 touches
// over all banks.  Rows past n_out are zero.
template <int KS>
constexpr int proj_pitch() { return 32 * KS + 16; }

template <int KS>
__global__ __launch_bounds__(kProjThreads, 1) void ln_proj_fwd_mfma(ProjProblem p, ProjFwdArgs a) {
  constexpr int C = 16 * KS;
  constexpr int PITCH = proj_pitch<KS>();
  extern __shared__ __align__(16) char lds[];
  float* s_gamma = reinterpret_cast<float*>(lds);
  float* s_beta = s_gamma + C;
  char* s_w = lds + 8 * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8 channels of each 16 this lane holds
  const int li = lane & 31;    // token slot in the tile
  const int stride = gridDim.x * kProjWaves;
  int tile = blockIdx.x * kProjWaves + wave;

  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  auto load_x = [&](int t, u32x4* dst) {
    const int64_t tok = t < p.tiles ? tile_token(p, t, li) : -1;
    if (tok >= 0) {
      const u32x4* src = reinterpret_cast<const u32x4*>(xg + tok * C + 8 * half);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[ks] = src[2 * ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[ks] = u32x4{0, 0, 0, 0};
    }
  };

  // The first tile's x is requested before the weight copy so both are in flight.
  u32x4 xr[KS];
  load_x(tile, xr);

  const int n_tiles_out = (p.n_out + 31) >> 5;
  {
    constexpr int CHUNKS = C / 8;  // 16-byte pieces per weight row
    const int total = n_tiles_out * 32 * CHUNKS;
    const uint16_t* wq = static_cast<const uint16_t*>(a.w_qkv);
    const uint16_t* wb = static_cast<const uint16_t*>(a.w_bias);
    for (int idx = tid; idx < total; idx += kProjThreads) {
      const int r = idx / CHUNKS;
      const int ch = idx - r * CHUNKS;
      u32x4 w = {0, 0, 0, 0};
      if (r < p.n_qkv)
        w = reinterpret_cast<const u32x4*>(wq + static_cast<int64_t>(r) * C)[ch];
      else if (r < p.n_out)
        w = reinterpret_cast<const u32x4*>(wb + static_cast<int64_t>(r - p.n_qkv) * C)[ch];
      *reinterpret_cast<u32x4*>(s_w + r * PITCH + 16 * ch) = w;
    }
    for (int c = tid; c < C; c += kProjThreads) {
      s_gamma[c] = a.gamma[c];
      s_beta[c] = a.beta[c];
    }
  }
  __syncthreads();
  // Wait for the first tile here, outside the loop: the loop then starts in the
  // same state on every trip, and the compiler's wait before the first use of x
  // does not also wait for the next tile's prefetch.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) pipe::retire(xr[ks]);

  const int hd = p.H * p.D;
  uint16_t* const qg = static_cast<uint16_t*>(a.q);
  uint16_t* const kg = static_cast<uint16_t*>(a.k);
  uint16_t* const vg = static_cast<uint16_t*>(a.v);
  uint16_t* biasg = static_cast<uint16_t*>(a.bias);
  constexpr float inv_c = 1.0f / C;

  for (; tile < p.tiles; tile += stride) {
    u32x4 xn[KS];
    load_x(tile + stride, xn);

    // Layer-norm statistics: this lane's C/2 channels, then its partner lane's.
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += lo_bf16(xr[ks][i]) + hi_bf16(xr[ks][i]);
    const float mean = pair_sum(s) * inv_c;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d0 = lo_bf16(xr[ks][i]) - mean, d1 = hi_bf16(xr[ks][i]) - mean;
        ss = fmaf(d0, d0, ss);
        ss = fmaf(d1, d1, ss);
      }
    const float rstd = rsqrtf(fmaf(pair_sum(ss), inv_c, p.eps));

    const int64_t tok = tile_token(p, tile, li);
    const int64_t bpos = (biasg && tok >= 0) ? bias_pos(p, tok) : 0;
    if (half == 0 && tok >= 0 && a.mean) {
      a.mean[tok] = mean;
      a.rstd[tok] = rstd;
    }

    // Normalised, affine, rounded to bf16: the B operand (k = channel, n = token).
    u32x4 yb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 16 * ks + 8 * half;
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(s_gamma + c0);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(s_gamma + c0 + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(s_beta + c0);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(s_beta + c0 + 4);
      const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      const float bb[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y0 = fmaf((lo_bf16(xr[ks][i]) - mean) * rstd, g[2 * i], bb[2 * i]);
        const float y1 = fmaf((hi_bf16(xr[ks][i]) - mean) * rstd, g[2 * i + 1], bb[2 * i + 1]);
        yb[ks][i] = pack_bf16(y0, y1);
      }
    }

    // Every weight tile: D[o][t] = sum_c W[o][c] y[t][c]; lane (li, half) then
    // holds outputs 8g + 4*half + 0..3 of token li in registers 4g..4g+3.
    for (int ot = 0; ot < n_tiles_out; ++ot) {
      const char* wrow = s_w + (ot * 32 + li) * PITCH + 16 * half;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mma(*reinterpret_cast<const u32x4*>(wrow + 32 * ks), yb[ks], acc);

      // Trade halves with the partner lane so each lane owns 8 consecutive
      // outputs of its token: the low half gets groups 1 and 3, the high half
      // groups 0 and 2.
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int g0 = 2 * pr, g1 = 2 * pr + 1;
        const uint32_t a0 = pack_bf16(acc[4 * g0], acc[4 * g0 + 1]), a1 = pack_bf16(acc[4 * g0 + 2], acc[4 * g0 + 3]);
        const uint32_t b0 = pack_bf16(acc[4 * g1], acc[4 * g1 + 1]), b1 = pack_bf16(acc[4 * g1 + 2], acc[4 * g1 + 3]);
        const auto r0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
        const u32x4 out = {r0[0], r1[0], r0[1], r1[1]};
        const int o8 = ot * 32 + 8 * (half ? g0 : g1);
        if (tok < 0) continue;
        if (o8 + 8 <= p.n_qkv) {
          const int which = o8 / hd;
          const int col = o8 - which * hd;
          uint16_t* dst = which == 0 ? qg : (which == 1 ? kg : vg);
          *reinterpret_cast<u32x4*>(dst + tok * hd + col) = out;
        } else if (o8 < p.n_out) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int hb = o8 + j - p.n_qkv;
            if (hb >= 0 && hb < p.H) {
              const uint32_t w = out[j >> 1];
              biasg[static_cast<int64_t>(hb) * p.T + bpos] = static_cast<uint16_t>((j & 1) ? (w >> 16) : (w & 0xffffu));
            }
          }
        }
      }
    }

#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xr[ks] = xn[ks];
  }
}

// ---------------------------------------------------------------- vector kernel

constexpr int kVecTokens = 8;
constexpr int kVecThreads = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One workgroup per 8 tokens: statistics per wave, the normalised tokens in
// LDS (rounded to the storage type), then one output per thread and step.
template <typename T>
__global__ __launch_bounds__(kVecThreads) void ln_proj_fwd_vector(ProjProblem p, ProjFwdArgs a) {
  extern __shared__ float ys[];  // [kVecTokens][C]
  const int C = p.C;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kVecTokens;
  const T* x = static_cast<const T*>(a.x);

  for (int ti = wave; ti < kVecTokens; ti += kVecThreads / 64) {
    const int64_t tok = t0 + ti;
    float* yt = ys + ti * C;
    if (tok >= p.T) {
      for (int c = lane; c < C; c += 64) yt[c] = 0.f;
      continue;
    }
    float s = 0.f;
    for (int c = lane; c < C; c += 64) {
      const float v = Elem<T>::load(x, tok * C + c);
      yt[c] = v;
      s += v;
    }
    const float mean = wave_sum(s) / C;
    float ss = 0.f;
    for (int c = lane; c < C; c += 64) {
      const float d = yt[c] - mean;
      ss = fmaf(d, d, ss);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(ss) / C + p.eps);
    for (int c = lane; c < C; c += 64) {
      const float y = fmaf((yt[c] - mean) * rstd, a.gamma[c], a.beta[c]);
      yt[c] = sizeof(T) == 2 ? bf16_to_f32(f32_to_bf16(y)) : y;
    }
    if (lane == 0 && a.mean) {
      a.mean[tok] = mean;
      a.rstd[tok] = rstd;
    }
  }
  __syncthreads();

  const int hd = p.H * p.D;
  const T* wq = static_cast<const T*>(a.w_qkv);
  const T* wb = static_cast<const T*>(a.w_bias);
  for (int idx = threadIdx.x; idx < kVecTokens * p.n_out; idx += kVecThreads) {
    const int ti = idx / p.n_out;
    const int o = idx - ti * p.n_out;
    const int64_t tok = t0 + ti;
    if (tok >= p.T) continue;
    const T* w = o < p.n_qkv ? wq + static_cast<int64_t>(o) * C : wb + static_cast<int64_t>(o - p.n_qkv) * C;
    const float* yt = ys + ti * C;
    float acc = 0.f;
    for (int c = 0; c < C; ++c) acc = fmaf(yt[c], Elem<T>::load(w, c), acc);
    if (o < p.n_qkv) {
      const int which = o / hd;
      T* dst = static_cast<T*>(which == 0 ? a.q : (which == 1 ? a.k : a.v));
      Elem<T>::store(dst, tok * hd + (o - which * hd), acc);
    } else {
      Elem<T>::store(static_cast<T*>(a.bias), bias_offset(p, o - p.n_qkv, tok), acc);
    }
  }
}

template <int KS>
size_t mfma_lds_bytes(const ProjProblem& p) {
  return 8 * 16 * KS + static_cast<size_t>((p.n_out + 31) / 32) * 32 * proj_pitch<KS>();
}

template <int KS>
hipError_t launch_mfma(const ProjProblem& p, const ProjFwdArgs& a, size_t lds, hipStream_t s) {
  auto kern = ln_proj_fwd_mfma<KS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kProjThreads, lds)) != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int want = (p.tiles + kProjWaves - 1) / kProjWaves;
  const int grid = want < cus * per_cu ? want : cus * per_cu;
  KernelTimer timer("ln_proj_fwd", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kProjThreads), lds, s, p, a);
  return hipGetLastError();
}

constexpr size_t kMaxLds = 160 * 1024;

}  // namespace

hipError_t launch_ln_proj_fwd(const ProjProblem& p, const ProjFwdArgs& a, hipStream_t s) {
  if (p.dtype == 1) {
    switch (p.C) {
      case 32: if (mfma_lds_bytes<2>(p) <= kMaxLds) return launch_mfma<2>(p, a, mfma_lds_bytes<2>(p), s); break;
      case 64: if (mfma_lds_bytes<4>(p) <= kMaxLds) return launch_mfma<4>(p, a, mfma_lds_bytes<4>(p), s); break;
      case 128: if (mfma_lds_bytes<8>(p) <= kMaxLds) return launch_mfma<8>(p, a, mfma_lds_bytes<8>(p), s); break;
      default: break;
    }
  }
  const size_t lds = static_cast<size_t>(kVecTokens) * p.C * sizeof(float);
  const int64_t grid = (p.T + kVecTokens - 1) / kVecTokens;
  KernelTimer timer("ln_proj_fwd_vector", s);
  if (p.dtype == 1)
    hipLaunchKernelGGL(ln_proj_fwd_vector<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
  else
    hipLaunchKernelGGL(ln_proj_fwd_vector<float>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
  return hipGetLastError();
}

}  // namespace evo
