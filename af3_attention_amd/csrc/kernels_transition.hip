// Fused SwiGLU transition, forward (MegaFold, gist.science technical summary,
// Methodik section 3 "EvoFusion": layer norm, linear projections and SwiGLU run
// as one operator, so intermediates are not materialised in HBM).
//
// For every token t of x [A, B, C], with y the layer norm of x:
//   a = y w_a^T, b = y w_b^T          (hidden = n*C units each)
//   h = silu(a) * b,  silu(a) = a / (1 + e^-a)
//   out = h w_out^T                    ([T, C])
// HBM sees x in and out (and the per-token statistics) out; y, a, b and h live
// in registers.
//
// bf16, C in {64, 128}.  A workgroup of 12 (C = 128) or 8 (C = 64) waves takes
// 384 or 256 tokens (one 32-token tile per wave) at a time and streams the
// weights through LDS in chunks of 64 hidden units (w_a and w_b rows, the
// matching w_out columns), double-buffered: every chunk is read once from L2 per
// pass, copied straight from global memory into LDS.  Per chunk and 32 hidden
// units a wave forms a and b on the matrix cores (D[hidden][token]), applies
// the gate in registers, and the packed accumulator registers are directly the
// B operand of out += w_out[:, chunk] h (the A operand reads w_out with the same
// permutation of the hidden index).

#include <hip/hip_runtime.h>

#include "evoattn_internal.h"
#include "mfma_common.h"
#include "pipe_common.h"
#include "proj_common.h"
#include "transition_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace trans;
using proj::hi_bf16;
using proj::lo_bf16;

// Waves per workgroup: 12 (three per SIMD) at C = 128, where the registers allow
// it and the third wave per SIMD hides latency that two do not; 8 at C = 64, where
// it measured slightly faster.
template <int KS>
constexpr int fwd_waves() { return KS == 8 ? 12 : 8; }

template <int KS>
__global__ __launch_bounds__(64 * fwd_waves<KS>(), 1) void transition_fwd_mfma(TransProblem p, TransFwdArgs a) {
  constexpr int kFwdWaves = fwd_waves<KS>();
  constexpr int kFwdThreads = 64 * kFwdWaves;
  using L = TransLayout<KS>;
  constexpr int C = L::C;
  constexpr int CT = C / 32;
  extern __shared__ __align__(16) char lds[];
  float* s_gamma = reinterpret_cast<float*>(lds);
  float* s_beta = s_gamma + C;
  char* wbuf = lds + 8 * C;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int nch = p.hidden / kHC;
  const int npass = (p.tiles + kFwdWaves - 1) / kFwdWaves;

  const int wave_u = pipe::wave_id();
  const uint32_t wbuf_a = pipe::lds_addr(wbuf);
  WeightCopy<KS, kFwdWaves> wc;
  wc.init(a.w_a, a.w_b, a.w_out, p.hidden, wave_u, lane);

  for (int c = tid; c < C; c += kFwdThreads) {
    s_gamma[c] = a.gamma[c];
    s_beta[c] = a.beta[c];
  }
  const int first = blockIdx.x;
  if (first < npass) wc.issue(0, wbuf_a, wave_u);
  pipe::wait_vmcnt<0>();
  __syncthreads();

  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  uint16_t* og = static_cast<uint16_t*>(a.out);
  constexpr float inv_c = 1.0f / C;
  int buf = 0;

  for (int pass = first; pass < npass; pass += gridDim.x) {
    const int64_t t = static_cast<int64_t>(pass * kFwdWaves + wave) * 32 + li;
    const bool valid = t < p.T;
    const int64_t tok = valid ? t : 0;

    // Layer norm of the tile's tokens (each token's channels on two lanes), as
    // the bf16 B operand y[k = channel][n = token].
    u32x4 yb[KS];
    {
      u32x4 xr[KS];
      const u32x4* src = reinterpret_cast<const u32x4*>(xg + tok * C + 8 * half);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xr[ks] = valid ? src[2 * ks] : u32x4{0, 0, 0, 0};
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
      if (half == 0 && valid && a.mean) {
        a.mean[tok] = mean;
        a.rstd[tok] = rstd;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 16 * ks + 8 * half;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y0 = fmaf((lo_bf16(xr[ks][i]) - mean) * rstd, s_gamma[c0 + 2 * i], s_beta[c0 + 2 * i]);
          const float y1 = fmaf((hi_bf16(xr[ks][i]) - mean) * rstd, s_gamma[c0 + 2 * i + 1], s_beta[c0 + 2 * i + 1]);
          yb[ks][i] = pack_bf16(y0, y1);
        }
      }
    }

    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};

    for (int ch = 0; ch < nch; ++ch) {
      // The next chunk of weights (of this pass, or the first of the next pass).
      const bool more = ch + 1 < nch || pass + static_cast<int>(gridDim.x) < npass;
      if (more) wc.issue(ch + 1 < nch ? ch + 1 : 0, wbuf_a + (buf ^ 1) * L::CHUNK, wave_u);
      const char* cw = wbuf + buf * L::CHUNK;
#pragma unroll
      for (int ht = 0; ht < kHC / 32; ++ht) {
        // a, b: D[hidden][token] for 32 hidden units.
        const char* ra = cw + L::WA + (32 * ht + li) * L::PW + 16 * half;
        const char* rb = cw + L::WB + (32 * ht + li) * L::PW + 16 * half;
        f32x16 fa = {}, fb = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          fa = mma(*reinterpret_cast<const u32x4*>(ra + 32 * ks), yb[ks], fa);
          fb = mma(*reinterpret_cast<const u32x4*>(rb + 32 * ks), yb[ks], fb);
        }
        // h = silu(a) * b, packed: registers 8kk..8kk+7 are the B operand of k-step kk
        // (hidden 32 ht + 16 kk + {4 half + 0..3, 8 + 4 half + 0..3}).
        u32x4 hb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int v = 8 * kk + 2 * i;
            hb[kk][i] = pack_bf16(silu(fa[v]) * fb[v], silu(fa[v + 1]) * fb[v + 1]);
          }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int j0 = 32 * ht + 16 * kk + 4 * half;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const char* ro = cw + L::WO + (32 * ct + li) * L::PO;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(ro + 2 * j0);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(ro + 2 * (j0 + 8));
            acc[ct] = mma(u32x4{lo[0], lo[1], hi[0], hi[1]}, hb[kk], acc[ct]);
          }
        }
      }
      // This wave's copies of the next chunk have landed; the barrier publishes
      // them and ends every wave's reads of this chunk.
      pipe::wait_vmcnt<0>();
      __syncthreads();
      buf ^= 1;
    }

    // out[token][c]: D[c][token]; trade halves with the partner lane for 16-byte stores.
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int g0 = 2 * pr, g1 = 2 * pr + 1;
        const f32x16& d = acc[ct];
        const uint32_t a0 = pack_bf16(d[4 * g0], d[4 * g0 + 1]), a1 = pack_bf16(d[4 * g0 + 2], d[4 * g0 + 3]);
        const uint32_t b0 = pack_bf16(d[4 * g1], d[4 * g1 + 1]), b1 = pack_bf16(d[4 * g1 + 2], d[4 * g1 + 3]);
        const auto r0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
        if (valid)
          *reinterpret_cast<u32x4*>(og + tok * C + 32 * ct + 8 * (half ? g0 : g1)) = u32x4{r0[0], r1[0], r0[1], r1[1]};
      }
  }
}

template <int KS>
hipError_t launch_fwd(const TransProblem& p, const TransFwdArgs& a, hipStream_t s) {
  using L = TransLayout<KS>;
  constexpr int kFwdWaves = fwd_waves<KS>();
  constexpr int kFwdThreads = 64 * kFwdWaves;
  auto kern = transition_fwd_mfma<KS>;
  const size_t lds = L::lds_bytes();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFwdThreads, lds)) != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int npass = (p.tiles + kFwdWaves - 1) / kFwdWaves;
  const int grid = npass < cus * per_cu ? npass : cus * per_cu;
  KernelTimer timer("transition_fwd", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFwdThreads), lds, s, p, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transition_fwd(const TransProblem& p, const TransFwdArgs& a, hipStream_t s) {
  if (p.C == 128) return launch_fwd<8>(p, a, s);
  if (p.C == 64) return launch_fwd<4>(p, a, s);
  return hipErrorInvalidValue;
}

}  // namespace evo
