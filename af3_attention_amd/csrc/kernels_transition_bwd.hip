// Backward of the fused SwiGLU transition (kernels_transition.hip).
//
// For L = sum out * dout, with y = xhat * gamma + beta the layer norm of x:
//   dh = dout w_out,  da = dh * b * silu'(a),  db = dh * silu(a)
//   dy = da w_a + db w_b,  dx = rstd (g - mean_c g - xhat mean_c(g xhat)), g = dy gamma
//   dw_out = dout^T h,  dw_a = da^T y,  dw_b = db^T y
// and, since y = xhat gamma + beta, with M_a = da^T xhat, s_a = sum_t da (and the
// same for b):  dw_a = M_a gamma + s_a (x) beta,
//   dgamma[c] = sum_j (w_a[j,c] M_a[j,c] + w_b[j,c] M_b[j,c])   (= sum_t dy xhat)
//   dbeta[c]  = sum_j (w_a[j,c] s_a[j] + w_b[j,c] s_b[j])       (= sum_t dy).
//
// Launches (bf16, C in {64, 128}):
//   1. dx, token by token: the forward's structure (256 tokens per workgroup,
//      weights streamed through LDS in 64-unit hidden chunks) recomputing a and b,
//      with dh = w_out^T dout, the gate's derivative in registers, and
//      dy += w_a^T da + w_b^T db read from the same LDS chunk transposed.
//   2. Weight-gradient partial sums over fixed token ranges, one workgroup per
//      (64-unit hidden group, token range): a, b and dh are recomputed with the
//      tokens on the accumulator rows, so da, db and h leave the registers as
//      operands whose contraction index is the token; they are exchanged through
//      LDS and accumulated into M_a, M_b and dout^T h against xhat and dout staged
//      per 64 tokens, by a second group of waves one chunk behind the first.  The
//      hidden groups of one range share an XCD.
//   3. Finalize: partials summed in fixed slots of ranges (each in increasing order), dw_a,
//      dw_b, dw_out, and dgamma / dbeta by fixed-shape sums.
// Nothing of size tokens x hidden is written to memory; every sum has a fixed order.

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
using pipe::lds_addr;
using pipe::lds_load_tr;
using pipe::xcd_logical_block;
using proj::hi_bf16;
using proj::lo_bf16;

constexpr int kTC = 64;          // tokens per staged chunk of the partial-sum kernel
constexpr int kMaxRanges = 64;   // token ranges of the partial sums (at most)
constexpr int kTargetBlocks = 256;  // one partial-sum workgroup per CU
constexpr int kFinThreads = 256;

__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.f + fast_exp2(-a * kLog2e)); }

// A operand read transposed from an LDS tile with `pitch` bytes per row:
// lane gets column c0 + lane % 32 at rows r0 + {4 half + 0..3, 8 + 4 half + 0..3},
// the row order of accumulator registers 8t..8t+7.
struct TrRead {
  int row, col;
  __device__ __forceinline__ explicit TrRead(int lane) {
    const int i16 = lane & 15;
    row = 4 * (lane >> 5) + (i16 >> 2);
    col = (lane & 16) + 4 * (i16 & 3);
  }
  __device__ __forceinline__ u32x4 operator()(uint32_t base, int pitch, int r0, int c0) const {
    const uint32_t ad = base + (r0 + row) * pitch + (c0 + col) * 2;
    const u32x2 lo = lds_load_tr(ad);
    const u32x2 hi = lds_load_tr(ad + 8 * pitch);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// ---------------------------------------------------------------- 1. dx

template <int KS>
__global__ __launch_bounds__(kThreads, 1) void transition_bwd_dx(TransProblem p, TransBwdArgs a, uint16_t* xh_out) {
  using L = TransLayout<KS>;
  constexpr int C = L::C;
  constexpr int CT = C / 32;
  extern __shared__ __align__(16) char lds[];
  float* s_gamma = reinterpret_cast<float*>(lds);
  float* s_beta = s_gamma + C;
  char* wbuf = lds + 8 * C;
  const uint32_t wbuf_a = lds_addr(wbuf);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int nch = p.hidden / kHC;
  const int npass = (p.tiles + kWaves - 1) / kWaves;
  const TrRead tr(lane);

  const int wave_u = pipe::wave_id();
  WeightCopy<KS> wc;
  wc.init(a.w_a, a.w_b, a.w_out, p.hidden, wave_u, lane);
  for (int c = tid; c < C; c += kThreads) {
    s_gamma[c] = a.gamma[c];
    s_beta[c] = a.beta[c];
  }
  const int first = blockIdx.x;
  if (first < npass) wc.issue(0, wbuf_a, wave_u);
  pipe::wait_vmcnt<0>();
  __syncthreads();

  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  const uint16_t* dog = static_cast<const uint16_t*>(a.dout);
  uint16_t* dxg = static_cast<uint16_t*>(a.dx);
  constexpr float inv_c = 1.0f / C;
  int buf = 0;

  for (int pass = first; pass < npass; pass += gridDim.x) {
    const int64_t t = static_cast<int64_t>(pass * kWaves + wave) * 32 + li;
    const bool valid = t < p.T;
    const int64_t tok = valid ? t : 0;
    const float mean = valid ? a.mean[tok] : 0.f;
    const float rstd = valid ? a.rstd[tok] : 0.f;

    // y as the B operand (k = channel, 8 consecutive per lane half), formed from
    // xhat rounded to bf16: that rounded xhat goes to the workspace, where the
    // weight-gradient pass stages it as it is and recomputes a and b from it, so
    // both passes start from the same xhat.  The workspace holds whole passes:
    // tokens past the end store their zeros there with no branch.  All x loads
    // precede the stores (which may alias them as far as the compiler knows), and
    // the stores drain under the first chunk's products.
    u32x4 yb[KS];
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(xg + tok * C + 8 * half);
      u32x4* xh_dst = reinterpret_cast<u32x4*>(xh_out + t * C + 8 * half);
      u32x4 xr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xr[ks] = src[2 * ks];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 16 * ks + 8 * half;
        u32x4 xh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h0 = (lo_bf16(xr[ks][i]) - mean) * rstd, h1 = (hi_bf16(xr[ks][i]) - mean) * rstd;
          xh[i] = pack_bf16(h0, h1);
          yb[ks][i] = pack_bf16(fmaf(lo_bf16(xh[i]), s_gamma[c0 + 2 * i], s_beta[c0 + 2 * i]),
                                fmaf(hi_bf16(xh[i]), s_gamma[c0 + 2 * i + 1], s_beta[c0 + 2 * i + 1]));
        }
        xh_dst[2 * ks] = xh;
      }
    }
    // dout as the B operand of dh, channels in accumulator-row order:
    // k-step ks holds 16 ks + {4 half + 0..3, 8 + 4 half + 0..3}.
    u32x4 db_op[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint16_t* row = dog + tok * C + 16 * ks + 4 * half;
      const u32x2 lo = valid ? *reinterpret_cast<const u32x2*>(row) : u32x2{0, 0};
      const u32x2 hi = valid ? *reinterpret_cast<const u32x2*>(row + 8) : u32x2{0, 0};
      db_op[ks] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }

    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};

    for (int ch = 0; ch < nch; ++ch) {
      // The next chunk (of this pass, or the first of the next) is copied into the
      // other buffer while this one is used.
      const bool more = ch + 1 < nch || pass + static_cast<int>(gridDim.x) < npass;
      if (more) wc.issue(ch + 1 < nch ? ch + 1 : 0, wbuf_a + (buf ^ 1) * L::CHUNK, wave_u);
      const char* cw = wbuf + buf * L::CHUNK;
      const uint32_t cwa = wbuf_a + buf * L::CHUNK;
#pragma unroll
      for (int ht = 0; ht < kHC / 32; ++ht) {
        // a, b, dh: D[hidden][token] for 32 hidden units.
        const char* ra = cw + L::WA + (32 * ht + li) * L::PW + 16 * half;
        const char* rb = cw + L::WB + (32 * ht + li) * L::PW + 16 * half;
        f32x16 fa = {}, fb = {}, fd = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          fa = mma(*reinterpret_cast<const u32x4*>(ra + 32 * ks), yb[ks], fa);
          fb = mma(*reinterpret_cast<const u32x4*>(rb + 32 * ks), yb[ks], fb);
          fd = mma(tr(cwa + L::WO, L::PO, 16 * ks, 32 * ht), db_op[ks], fd);
          // keeps the compiler from hoisting every k-step's LDS reads (registers)
          __builtin_amdgcn_sched_barrier(0);
        }
        // da = dh b silu'(a), db = dh silu(a); packed registers 8kk..8kk+7 are the
        // B operand of k-step kk over hidden 32 ht + 16 kk + (accumulator-row order).
        u32x4 dab[2], dbb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float va[2], vb[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int v = 8 * kk + 2 * i + e;
              // silu(a) = a s, silu'(a) = s (1 + a (1 - s)) = s + silu(a) (1 - s)
              const float s = sigmoid_f(fa[v]);
              const float sl = fa[v] * s;
              va[e] = fd[v] * fb[v] * fmaf(-sl, s, s + sl);
              vb[e] = fd[v] * sl;
            }
            dab[kk][i] = pack_bf16(va[0], va[1]);
            dbb[kk][i] = pack_bf16(vb[0], vb[1]);
          }
        // dy[c][token] += w_a^T da + w_b^T db: A = w^T[c][hidden] read transposed.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            acc[ct] = mma(tr(cwa + L::WA, L::PW, 32 * ht + 16 * kk, 32 * ct), dab[kk], acc[ct]);
            acc[ct] = mma(tr(cwa + L::WB, L::PW, 32 * ht + 16 * kk, 32 * ct), dbb[kk], acc[ct]);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      pipe::wait_vmcnt<0>();
      __syncthreads();
      buf ^= 1;
    }

    // Layer-norm backward on the token's channels (32 ct + 8 g + 4 half + 0..3).
    u32x2 xd[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        xd[ct][g] = valid ? *reinterpret_cast<const u32x2*>(xg + tok * C + 32 * ct + 8 * g + 4 * half) : u32x2{0, 0};
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 32 * ct + 8 * g + 4 * half + e;
          const uint32_t u = xd[ct][g][e >> 1];
          const float xh = (((e & 1) ? hi_bf16(u) : lo_bf16(u)) - mean) * rstd;
          const float gv = acc[ct][4 * g + e] * s_gamma[c];
          acc[ct][4 * g + e] = gv;
          s1 += gv;
          s2 = fmaf(gv, xh, s2);
        }
    s1 = pair_sum(s1) * inv_c;
    s2 = pair_sum(s2) * inv_c;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = xd[ct][g][e >> 1];
          const float xh = (((e & 1) ? hi_bf16(u) : lo_bf16(u)) - mean) * rstd;
          acc[ct][4 * g + e] = rstd * (acc[ct][4 * g + e] - s1 - xh * s2);
        }
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
          *reinterpret_cast<u32x4*>(dxg + tok * C + 32 * ct + 8 * (half ? g0 : g1)) = u32x4{r0[0], r1[0], r0[1], r1[1]};
      }
  }
}

// ---------------------------------------------------------------- 2. weight-gradient partials

template <int KS>
struct WLayout {
  using L = TransLayout<KS>;
  static constexpr int C = L::C;
  static constexpr int PX = 2 * C + 32;                 // staged token row (xhat or dout), bytes
  static constexpr int STAGE = 2 * kTC * PX;            // xhat then dout of one chunk
  static constexpr int NSTAGE = 3;                      // chunks being read by C, read by A, written
  static constexpr int XCH = 4 * 3 * 2 * 64 * 16;       // exchange: job x (da, db, h) x k-step x lane
  static constexpr int S0 = 0;
  static constexpr int X0 = S0 + NSTAGE * STAGE;        // two exchange buffers
  static constexpr int SUMS = X0 + 2 * XCH;             // 4 jobs x 2 x 32 floats
  static constexpr size_t bytes() { return static_cast<size_t>(SUMS) + 4 * 2 * 32 * 4; }
};

// One workgroup per (64-unit hidden group, token range); the range's tokens are
// taken in chunks of 64 by two groups of waves, one chunk apart:
//   waves 0..3 (phase A, chunk s + 1): job (32 hidden units ht, 32 tokens sub)
//     forms a, b, dh as D[token][hidden] from the staged xhat and dout rows against
//     weights held in registers, with gamma folded in: a = xhat (w_a diag(gamma))^T
//     + w_a beta (and the same for b), then da, db, h, packed as operands whose
//     contraction index is the token, go to an exchange buffer;
//   waves 4..7 (phase C, chunk s): the product tiles M_a += da^T xhat,
//     M_b += db^T xhat, Mo += dout^T h over the chunk's 64 tokens, then they stage
//     chunk s + 2 (xhat rows written by the dx pass, and dout), loaded one step
//     earlier so that the loads overlap a barrier and a phase C.
// Three stages and two exchange buffers: one barrier per step.
template <int KS>
__global__ __launch_bounds__(kThreads, 1) void transition_bwd_wpart(TransProblem p, TransBwdArgs a, int ngroups,
                                                                   int ranges, int range_chunks, const uint16_t* xh,
                                                                   float* ma, float* mb, float* mo, float* sa,
                                                                   float* sb) {
  using L = TransLayout<KS>;
  using W = WLayout<KS>;
  constexpr int C = L::C;
  constexpr int CT = C / 32;
  constexpr int PX = W::PX;
  constexpr int XPL = C / 8;                     // 16-byte pieces per token row
  constexpr int CTHREADS = kThreads / 2;         // threads of the phase-C waves
  constexpr int NPC = kTC * XPL / CTHREADS;      // pieces of each tensor per phase-C thread
  constexpr int NT = 3 * 2 * CT;                 // product tiles per workgroup
  constexpr int TPW = NT / 4;                    // per phase-C wave
  static_assert(kTC * XPL % CTHREADS == 0 && NT % 4 == 0, "work must divide evenly");
  static_assert((2 * CT) % 4 == 0, "a phase-C wave's i-th tile has the same quantity for every wave");
  extern __shared__ __align__(16) char lds[];
  const uint32_t base = lds_addr(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = pipe::wave_id();
  const int half = lane >> 5;
  const int li = lane & 31;
  const TrRead tr(lane);
  const int blk = xcd_logical_block(blockIdx.x, ngroups * ranges);
  const int group = blk % ngroups;
  const int range = blk / ngroups;
  const int h0 = group * kHC;
  const int64_t t_begin = static_cast<int64_t>(range) * range_chunks * kTC;
  const int64_t t_end = min(p.T, t_begin + static_cast<int64_t>(range_chunks) * kTC);
  const int nch = static_cast<int>((t_end - t_begin + kTC - 1) / kTC);
  const bool is_a = wave < 4;

  auto stage_x = [&](int c) { return base + W::S0 + (c % W::NSTAGE) * W::STAGE; };
  // Exchange slot of (chunk parity, job, quantity 0 da / 1 db / 2 h, k-step) for one lane.
  auto xslot = [&](int c, int job, int q, int kk) {
    return W::X0 + (c & 1) * W::XCH + ((job * 3 + q) * 2 + kk) * 1024 + 16 * lane;
  };

  // ---- staging (phase-C waves): chunk c's xhat and dout rows, in registers then LDS
  const uint16_t* dog = static_cast<const uint16_t*>(a.dout);
  const int ctid = tid - CTHREADS;
  u32x4 xr[NPC], dr[NPC];
  // Tokens past the range are loaded from its last token (no branch around the
  // loads) and staged as zeros.
  // Addresses are a uniform base (the chunk's first token) plus 32-bit lane offsets.
  auto stage_load = [&](int c) {
    const int64_t t0 = t_begin + static_cast<int64_t>(c) * kTC;
    const char* xb = reinterpret_cast<const char*>(pipe::uniform_ptr(xh + t0 * C));
    const char* db = reinterpret_cast<const char*>(pipe::uniform_ptr(dog + t0 * C));
    const int tmax = static_cast<int>(t_end - 1 - t0);
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int idx = ctid + i * CTHREADS;
      const int t = min(idx / XPL, tmax), jj = idx - (idx / XPL) * XPL;
      const uint32_t off = static_cast<uint32_t>(t * (2 * C) + 16 * jj);
      xr[i] = *reinterpret_cast<const u32x4*>(xb + off);
      dr[i] = *reinterpret_cast<const u32x4*>(db + off);
    }
  };
  auto stage_store = [&](int c) {
    char* sx = lds + (stage_x(c) - base);
    char* sd = sx + kTC * PX;
    const int64_t t0 = t_begin + static_cast<int64_t>(c) * kTC;
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int idx = ctid + i * CTHREADS;
      const int t = idx / XPL, jj = idx - (idx / XPL) * XPL;
      const bool in = t0 + t < t_end;
      *reinterpret_cast<u32x4*>(sx + t * PX + 16 * jj) = in ? xr[i] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(sd + t * PX + 16 * jj) = in ? dr[i] : u32x4{0, 0, 0, 0};
    }
  };

  // The two groups run separate loops (disjoint registers) that meet at the same
  // barriers: two in the prologue, one per step, one before the range sums.
  float* sums = reinterpret_cast<float*>(lds + W::SUMS);  // [job][a/b][32]
  if (is_a) {
    // Phase-A state: this lane's hidden unit j (B-operand column), its weights over
    // the k slots 16 ks + 8 half + 0..7 (w_a, w_b scaled by gamma; w_out as is),
    // and the constants w_a beta, w_b beta.
    const int ht = wave & 1, sub = wave >> 1;
    u32x4 wa_op[KS], wb_op[KS], wo_op[KS];
    float ca = 0.f, cb = 0.f;
    {
      const int j = h0 + 32 * ht + li;
      const uint16_t* wa_g = static_cast<const uint16_t*>(a.w_a) + static_cast<int64_t>(j) * C;
      const uint16_t* wb_g = static_cast<const uint16_t*>(a.w_b) + static_cast<int64_t>(j) * C;
      const uint16_t* wo_g = static_cast<const uint16_t*>(a.w_out);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 16 * ks + 8 * half;
        const u32x4 ra = *reinterpret_cast<const u32x4*>(wa_g + c0);
        const u32x4 rb = *reinterpret_cast<const u32x4*>(wb_g + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = c0 + 2 * i;
          const float g0 = a.gamma[c], g1 = a.gamma[c + 1], b0 = a.beta[c], b1 = a.beta[c + 1];
          const float a0 = lo_bf16(ra[i]), a1 = hi_bf16(ra[i]), e0 = lo_bf16(rb[i]), e1 = hi_bf16(rb[i]);
          wa_op[ks][i] = pack_bf16(a0 * g0, a1 * g1);
          wb_op[ks][i] = pack_bf16(e0 * g0, e1 * g1);
          ca = fmaf(a0, b0, ca);
          ca = fmaf(a1, b1, ca);
          cb = fmaf(e0, b0, cb);
          cb = fmaf(e1, b1, cb);
          wo_op[ks][i] = static_cast<uint32_t>(wo_g[static_cast<int64_t>(c) * p.hidden + j]) |
                         (static_cast<uint32_t>(wo_g[static_cast<int64_t>(c + 1) * p.hidden + j]) << 16);
        }
      }
      ca = pair_sum(ca);
      cb = pair_sum(cb);
    }
    float sacc = 0.f, sbcc = 0.f;  // per-lane partial sums of da and db

    // Phase A of chunk c: a, b, dh for (ht, sub), then da, db, h to the exchange.
    auto phase_a = [&](int c) {
      const uint32_t sx = stage_x(c), sd = sx + kTC * PX;
      const uint32_t row = (sub * 32 + li) * PX + 16 * half;
      f32x16 fa, fb, fd = {};
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        fa[v] = ca;
        fb[v] = cb;
      }
      // Every operand read of the chunk is issued before the products, so that
      // the reads' latency is paid once.
      u32x4 xo[KS], dq[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        xo[ks] = pipe::lds_load16(sx + row + 32 * ks);
        dq[ks] = pipe::lds_load16(sd + row + 32 * ks);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        fa = mma(xo[ks], wa_op[ks], fa);
        fb = mma(xo[ks], wb_op[ks], fb);
        fd = mma(dq[ks], wo_op[ks], fd);
      }
      // Lane: hidden 32 ht + lane % 32; register v: token sub * 32 + accumulator row
      // v.  Tokens past the range hold xhat = dout = 0: dh = 0, so da = db = 0 there.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 oa, ob, oh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float va[2], vb[2], vh[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int v = 8 * kk + 2 * i + e;
            // silu(a) = a s, silu'(a) = s + silu(a) (1 - s)
            const float sg = sigmoid_f(fa[v]);
            const float sl = fa[v] * sg;
            va[e] = fd[v] * fb[v] * fmaf(-sl, sg, sg + sl);
            vb[e] = fd[v] * sl;
            vh[e] = sl * fb[v];
            sacc += va[e];
            sbcc += vb[e];
          }
          oa[i] = pack_bf16(va[0], va[1]);
          ob[i] = pack_bf16(vb[0], vb[1]);
          oh[i] = pack_bf16(vh[0], vh[1]);
        }
        *reinterpret_cast<u32x4*>(lds + xslot(c, wave, 0, kk)) = oa;
        *reinterpret_cast<u32x4*>(lds + xslot(c, wave, 1, kk)) = ob;
        *reinterpret_cast<u32x4*>(lds + xslot(c, wave, 2, kk)) = oh;
      }
    };

    __syncthreads();  // chunk 0 staged
    phase_a(0);
    __syncthreads();
    for (int s = 0; s < nch; ++s) {
      if (s + 1 < nch) phase_a(s + 1);
      __syncthreads();
    }
    const float ta = pair_sum(sacc), tb = pair_sum(sbcc);
    if (half == 0) {
      sums[(wave * 2 + 0) * 32 + li] = ta;
      sums[(wave * 2 + 1) * 32 + li] = tb;
    }
  } else {
    // Phase C of chunk c over the chunk's 64 tokens (four 16-token k-steps).  Wave
    // cw owns tiles cw + 4 i of the list (M_a tiles, M_b tiles, Mo tiles, 2 CT
    // each): i < CT / 2 are M_a tiles, their M_b partners are i + CT / 2, and the Mo
    // tiles of the same hidden half are i + CT.  Each group's operand reads are
    // issued before its products.
    const int cw = wave - 4;
    f32x16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
    // Every tile of this wave has the channel block ct = cw % CT ((cw + 4 i) % CT,
    // with CT in {2, 4}), so each k-step's xhat and dout operands are read once and
    // serve all of the wave's tiles of that k-step.
    auto phase_c = [&](int c) {
      const uint32_t sx = stage_x(c), sd = sx + kTC * PX;
      const int ct = cw % CT;
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {  // token halves: k-steps 2 hk, 2 hk + 1
        u32x4 xop[2], dop[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          xop[kk] = tr(sx, PX, 32 * hk + 16 * kk, 32 * ct);
          dop[kk] = tr(sd, PX, 32 * hk + 16 * kk, 32 * ct);
        }
#pragma unroll
        for (int pr = 0; pr < CT / 2; ++pr) {
          const int tht = (cw + 4 * pr) / CT;
          const int job = tht + 2 * hk;
          u32x4 av[2], bv[2], hv[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            av[kk] = *reinterpret_cast<const u32x4*>(lds + xslot(c, job, 0, kk));
            bv[kk] = *reinterpret_cast<const u32x4*>(lds + xslot(c, job, 1, kk));
            hv[kk] = *reinterpret_cast<const u32x4*>(lds + xslot(c, job, 2, kk));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            // M_a, M_b [hidden][c] += (da, db)[hidden][token] xhat[token][c]
            acc[pr] = mma(av[kk], xop[kk], acc[pr]);
            acc[pr + CT / 2] = mma(bv[kk], xop[kk], acc[pr + CT / 2]);
            // Mo[c][hidden] += dout[token][c]^T h[token][hidden]
            acc[CT + pr] = mma(dop[kk], hv[kk], acc[CT + pr]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Chunk c is loaded during step c - 3 (after that step's store) and staged
    // during step c - 2, so its loads have a barrier and a phase C to land.
    stage_load(0);
    stage_store(0);
    __syncthreads();
    if (nch > 1) {
      stage_load(1);
      stage_store(1);
    }
    if (nch > 2) stage_load(2);
    __syncthreads();
    for (int s = 0; s < nch; ++s) {
      phase_c(s);
      if (s + 2 < nch) stage_store(s + 2);
      if (s + 3 < nch) stage_load(s + 3);
      __syncthreads();
    }
    // Partial sums of this range: M_a, M_b [hidden][C], Mo [C][hidden].
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int q = (4 * i) / (2 * CT);
      const int rem = cw + 4 * i - q * (2 * CT);
      const int tht = rem / CT, ct = rem - (rem / CT) * CT;
      if (q < 2) {
        float* dst = (q == 0 ? ma : mb) + (static_cast<int64_t>(range) * p.hidden + h0 + 32 * tht) * C + 32 * ct + li;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[static_cast<int64_t>(acc_row(v, lane)) * C] = acc[i][v];
      } else {
        float* dst = mo + (static_cast<int64_t>(range) * C + 32 * ct) * p.hidden + h0 + 32 * tht + li;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[static_cast<int64_t>(acc_row(v, lane)) * p.hidden] = acc[i][v];
      }
    }
  }
  __syncthreads();
  // Range sums s_a, s_b [hidden]: jobs tht (tokens 0..31 of each chunk) then tht + 2.
  if (tid < kHC) {
    const int tht = tid >> 5, l = tid & 31;
    sa[static_cast<int64_t>(range) * p.hidden + h0 + tid] =
        sums[(tht * 2 + 0) * 32 + l] + sums[((tht + 2) * 2 + 0) * 32 + l];
    sb[static_cast<int64_t>(range) * p.hidden + h0 + tid] =
        sums[(tht * 2 + 1) * 32 + l] + sums[((tht + 2) * 2 + 1) * 32 + l];
  }
}

// ---------------------------------------------------------------- 3. finalize

__device__ __forceinline__ float bf(const void* p, int64_t i) { return bf16_to_f32(static_cast<const uint16_t*>(p)[i]); }

// 1024 threads = 8 slots x 128 columns: slot k sums ranges k, k + 8, ... in
// increasing order (its loads all in flight), then the slot sums are added in
// slot order.
constexpr int kSlots = 8;
constexpr int kCols = 128;
constexpr int kRowThreads = kSlots * kCols;

// One workgroup per hidden unit j: M_a, M_b, s_a, s_b over the ranges, dw_a, dw_b,
// and the products whose sums over j are dgamma and dbeta.
__global__ __launch_bounds__(kRowThreads) void transition_fin_hidden(TransProblem p, TransBwdArgs a, int ranges,
                                                                    const float* ma, const float* mb, const float* sa,
                                                                    const float* sb, float* tg, float* tb) {
  __shared__ float part[2][kSlots][kCols];
  __shared__ float s_r[2][kRowThreads / 2];
  __shared__ float s_sh[2];
  const int j = blockIdx.x;
  const int slot = threadIdx.x / kCols, cl = threadIdx.x - slot * kCols;
  // s_a, s_b: every range's partial loaded at once, then summed in range order.
  for (int r = threadIdx.x; r < 2 * ranges; r += kRowThreads) {
    const int q = r / ranges, rr = r - q * ranges;
    s_r[q][rr] = (q == 0 ? sa : sb)[static_cast<int64_t>(rr) * p.hidden + j];
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    float s = 0.f;
    for (int r = 0; r < ranges; ++r) s += s_r[threadIdx.x][r];
    s_sh[threadIdx.x] = s;
  }
  const int64_t rstride = static_cast<int64_t>(p.hidden) * p.C;
  for (int c0 = 0; c0 < p.C; c0 += kCols) {
    const int c = c0 + cl;
    float m_a = 0.f, m_b = 0.f;
    if (c < p.C) {
      const int64_t off = static_cast<int64_t>(j) * p.C + c;
#pragma unroll 8
      for (int r = slot; r < ranges; r += kSlots) {
        m_a += ma[r * rstride + off];
        m_b += mb[r * rstride + off];
      }
    }
    part[0][slot][cl] = m_a;
    part[1][slot][cl] = m_b;
    __syncthreads();
    if (slot == 0 && c < p.C) {
      m_a = part[0][0][cl];
      m_b = part[1][0][cl];
#pragma unroll
      for (int k = 1; k < kSlots; ++k) {
        m_a += part[0][k][cl];
        m_b += part[1][k][cl];
      }
      const float s_a = s_sh[0], s_b = s_sh[1];
      const int64_t off = static_cast<int64_t>(j) * p.C + c;
      a.dw_a[off] = fmaf(m_a, a.gamma[c], s_a * a.beta[c]);
      a.dw_b[off] = fmaf(m_b, a.gamma[c], s_b * a.beta[c]);
      const float wa = bf(a.w_a, off), wb = bf(a.w_b, off);
      tg[off] = fmaf(wa, m_a, wb * m_b);
      tb[off] = fmaf(wa, s_a, wb * s_b);
    }
    __syncthreads();
  }
}

// One workgroup per channel c: dw_out[c][:] over the ranges (the same slots).
__global__ __launch_bounds__(kRowThreads) void transition_fin_out(TransProblem p, TransBwdArgs a, int ranges,
                                                                 const float* mo) {
  __shared__ float part[kSlots][kCols];
  const int c = blockIdx.x;
  const int slot = threadIdx.x / kCols, cl = threadIdx.x - slot * kCols;
  const int64_t rstride = static_cast<int64_t>(p.C) * p.hidden;
  for (int j0 = 0; j0 < p.hidden; j0 += kCols) {
    const int j = j0 + cl;
    float s = 0.f;
    if (j < p.hidden) {
      const float* src = mo + static_cast<int64_t>(c) * p.hidden + j;
#pragma unroll 8
      for (int r = slot; r < ranges; r += kSlots) s += src[r * rstride];
    }
    part[slot][cl] = s;
    __syncthreads();
    if (slot == 0 && j < p.hidden) {
      s = part[0][cl];
#pragma unroll
      for (int k = 1; k < kSlots; ++k) s += part[k][cl];
      a.dw_out[static_cast<int64_t>(c) * p.hidden + j] = s;
    }
    __syncthreads();
  }
}

// One workgroup per channel c: dgamma, dbeta as sums over hidden units (thread i
// takes i, i + 256, ... in order, then a fixed pairwise tree).
__global__ __launch_bounds__(kFinThreads) void transition_fin_cols(TransProblem p, TransBwdArgs a, const float* tg,
                                                                  const float* tb) {
  __shared__ float sg[kFinThreads], sbb[kFinThreads];
  const int c = blockIdx.x;
  float g = 0.f, b = 0.f;
  for (int j = threadIdx.x; j < p.hidden; j += kFinThreads) {
    g += tg[static_cast<int64_t>(j) * p.C + c];
    b += tb[static_cast<int64_t>(j) * p.C + c];
  }
  sg[threadIdx.x] = g;
  sbb[threadIdx.x] = b;
  __syncthreads();
  for (int w = kFinThreads / 2; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) {
      sg[threadIdx.x] += sg[threadIdx.x + w];
      sbb[threadIdx.x] += sbb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.dgamma[c] = sg[0];
    a.dbeta[c] = sbb[0];
  }
}

// ---------------------------------------------------------------- launch

struct TWs {
  int ranges, range_chunks;
  size_t ma, mb, mo, sa, sb, tg, tb, xh, total;
};

TWs tws(const TransProblem& p) {
  TWs w{};
  // Enough ranges that (hidden groups x ranges) fills the CUs once.
  const int64_t chunks = (p.T + kTC - 1) / kTC;
  const int64_t groups = p.hidden / kHC;
  int64_t r = (kTargetBlocks + groups - 1) / groups;
  r = r < kMaxRanges ? r : kMaxRanges;
  r = r < chunks ? r : chunks;
  const int64_t per = (chunks + r - 1) / r;
  r = (chunks + per - 1) / per;
  w.ranges = static_cast<int>(r);
  w.range_chunks = static_cast<int>(per);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t hc = static_cast<size_t>(p.hidden) * p.C * sizeof(float);
  const size_t h = static_cast<size_t>(p.hidden) * sizeof(float);
  w.ma = 0;
  w.mb = up(w.ma + r * hc);
  w.mo = up(w.mb + r * hc);
  w.sa = up(w.mo + r * hc);
  w.sb = up(w.sa + r * h);
  w.tg = up(w.sb + r * h);
  w.tb = up(w.tg + hc);
  w.xh = up(w.tb + hc);
  // xhat rows for every token slot of the dx kernel's passes (kWaves x 32 tokens each)
  const size_t slots = static_cast<size_t>((p.tiles + kWaves - 1) / kWaves) * kWaves * 32;
  w.total = up(w.xh + slots * p.C * sizeof(uint16_t));
  return w;
}

template <typename K>
hipError_t grid_for(K kern, size_t lds, int want, int* grid) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds)) != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  *grid = want < cus * per_cu ? want : cus * per_cu;
  return hipSuccess;
}

template <int KS>
hipError_t launch_bwd(const TransProblem& p, const TransBwdArgs& a, char* ws, hipStream_t s) {
  const TWs w = tws(p);
  hipError_t e;
  {
    const size_t lds = TransLayout<KS>::lds_bytes();
    int grid = 0;
    if ((e = grid_for(transition_bwd_dx<KS>, lds, (p.tiles + kWaves - 1) / kWaves, &grid)) != hipSuccess) return e;
    KernelTimer timer("transition_bwd_dx", s);
    hipLaunchKernelGGL(transition_bwd_dx<KS>, dim3(grid), dim3(kThreads), lds, s, p, a,
                       reinterpret_cast<uint16_t*>(ws + w.xh));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const size_t lds = WLayout<KS>::bytes();
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(transition_bwd_wpart<KS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int ngroups = p.hidden / kHC;
    KernelTimer timer("transition_bwd_wpart", s);
    hipLaunchKernelGGL(transition_bwd_wpart<KS>, dim3(ngroups * w.ranges), dim3(kThreads), lds, s, p, a, ngroups,
                       w.ranges, w.range_chunks, reinterpret_cast<const uint16_t*>(ws + w.xh),
                       reinterpret_cast<float*>(ws + w.ma),
                       reinterpret_cast<float*>(ws + w.mb), reinterpret_cast<float*>(ws + w.mo),
                       reinterpret_cast<float*>(ws + w.sa), reinterpret_cast<float*>(ws + w.sb));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  KernelTimer timer("transition_bwd_finalize", s);
  hipLaunchKernelGGL(transition_fin_hidden, dim3(p.hidden), dim3(kRowThreads), 0, s, p, a, w.ranges,
                     reinterpret_cast<const float*>(ws + w.ma), reinterpret_cast<const float*>(ws + w.mb),
                     reinterpret_cast<const float*>(ws + w.sa), reinterpret_cast<const float*>(ws + w.sb),
                     reinterpret_cast<float*>(ws + w.tg), reinterpret_cast<float*>(ws + w.tb));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(transition_fin_out, dim3(p.C), dim3(kRowThreads), 0, s, p, a, w.ranges,
                     reinterpret_cast<const float*>(ws + w.mo));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(transition_fin_cols, dim3(p.C), dim3(kFinThreads), 0, s, p, a,
                     reinterpret_cast<const float*>(ws + w.tg), reinterpret_cast<const float*>(ws + w.tb));
  return hipGetLastError();
}

}  // namespace

size_t transition_bwd_workspace_bytes(const TransProblem& p) { return tws(p).total; }

hipError_t launch_transition_bwd(const TransProblem& p, const TransBwdArgs& a, void* ws, hipStream_t s) {
  if (p.C == 128) return launch_bwd<8>(p, a, static_cast<char*>(ws), s);
  if (p.C == 64) return launch_bwd<4>(p, a, static_cast<char*>(ws), s);
  return hipErrorInvalidValue;
}

}  // namespace evo
