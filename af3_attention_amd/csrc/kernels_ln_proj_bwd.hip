// Backward of the fused layer norm + projections (kernels_ln_proj.hip).
//
// With G[t][o] the upstream gradient of output o of token t (dq | dk | dv rows,
// then the pair-bias heads gathered from dbias), the chain rule gives
//   dy[t][c]  = sum_o G[t][o] W[o][c]
//   dx[t][c]  = rstd_t (g - mean_c(g) - xhat mean_c(g xhat)),   g = dy * gamma
// and, with M[o][c] = sum_t G[t][o] xhat[t][c] and s[o] = sum_t G[t][o]
// (y = xhat * gamma + beta, so the sums over tokens factor through M and s):
//   dW[o][c]  = M[o][c] gamma[c] + s[o] beta[c]      (= sum_t G[t][o] y[t][c])
//   dgamma[c] = sum_o W[o][c] M[o][c]                  (= sum_t dy[t][c] xhat[t][c])
//   dbeta[c]  = sum_o W[o][c] s[o]                     (= sum_t dy[t][c])
//
// Launches:
//   1. dx, token by token: the forward's structure with outputs and channels
//      swapped (W^T resident in LDS, G streamed from HBM as the MFMA operand,
//      the layer-norm backward on registers; each token's channels sit on two lanes).
//   2. Partial M and s over fixed token ranges: one workgroup per (group of four
//      32-output tiles, token range); G and xhat are staged in LDS per 128 tokens
//      and read back transposed so that tokens are the contraction index.  The
//      groups of one range run on one XCD, so x is fetched from HBM once.
//   3. Finalize: partials summed in increasing range order, dW, the products
//      W*M and W*s, then their sums over o in increasing order.
// Every sum has a fixed order: results are bit-identical across calls.
//
// bf16 with C in {32, 64, 128} uses MFMA kernels for 1 and 2; fp32 and other
// channel counts use vector kernels with the same partial-sum layout.

#include <hip/hip_runtime.h>

#include "evoattn_internal.h"
#include "mfma_common.h"
#include "pipe_common.h"
#include "proj_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace proj;
using pipe::lds_addr;
using pipe::lds_load_tr;
using pipe::xcd_logical_block;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 128;      // tokens per staged chunk of the partial-sum kernel
constexpr int kGroupOut = 128;   // outputs per group (four 32-output tiles)
constexpr int kMaxRanges = 64;   // token ranges of the partial sums
constexpr size_t kMaxLds = 160 * 1024;

// Rows of the partial-M array: outputs padded to whole 32-output tiles.
__host__ __device__ __forceinline__ int padded_outputs(const ProjProblem& p) { return (p.n_out + 31) / 32 * 32; }

// Number of token ranges and kChunk-token chunks per range.
void range_split(const ProjProblem& p, int* ranges, int* range_chunks) {
  const int64_t chunks = (p.T + kChunk - 1) / kChunk;
  int64_t r = chunks < kMaxRanges ? chunks : kMaxRanges;
  const int64_t per = (chunks + r - 1) / r;
  r = (chunks + per - 1) / per;  // every range holds at least one token
  *ranges = static_cast<int>(r);
  *range_chunks = static_cast<int>(per);
}

// Width of the token-order pair-bias gradient buffer: H rounded up to 16, so
// that every 16-output k-step over it is one full load per lane.
__host__ __device__ __forceinline__ int bias_width(const ProjProblem& p) {
  return p.n_out > p.n_qkv ? (p.H + 15) / 16 * 16 : 0;
}

// Source of the 8 upstream gradients G[tok][o0 .. o0+7] (o0 a multiple of 8) as
// one 16-byte bf16 load: a dq/dk/dv row, or the token-order bias buffer gb
// [T][bias_width] (written by bias_grad_tokens), or nothing (zero).
struct GSource {
  const uint16_t* base;  // element (tok, o0) at base + tok * pitch
  int pitch;
  bool ok;               // false past the outputs: base is x (always present), values are 0
};
__device__ __forceinline__ GSource g_source(const ProjProblem& p, const ProjBwdArgs& a, const uint16_t* gb,
                                            int o0) {
  const int hd = p.H * p.D;
  if (o0 < p.n_qkv) {
    const int which = o0 / hd;
    const uint16_t* src = static_cast<const uint16_t*>(which == 0 ? a.dq : (which == 1 ? a.dk : a.dv));
    return GSource{src + (o0 - which * hd), hd, true};
  }
  const int hb = bias_width(p);
  if (o0 < p.n_qkv + hb) return GSource{gb + (o0 - p.n_qkv), hb, true};
  return GSource{static_cast<const uint16_t*>(a.x), 0, false};  // x is always present
}
// Loaded unconditionally (no branch around the load); the caller applies ok.
__device__ __forceinline__ u32x4 g_load(const GSource& g, int64_t tok) {
  return *reinterpret_cast<const u32x4*>(g.base + tok * g.pitch);
}

// The pair-bias gradient (fp32, [H][A][B] in the attention's frame) in token
// order as bf16, zero-padded to bias_width: one thread per token.
__global__ __launch_bounds__(256) void bias_grad_tokens(ProjProblem p, ProjBwdArgs a, uint16_t* gb) {
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (tok >= p.T) return;
  const int hb = bias_width(p);
  const float* src = a.dbias + bias_pos(p, tok);
  for (int h0 = 0; h0 < hb; h0 += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = h0 + e < p.H ? src[static_cast<int64_t>(h0 + e) * p.T] : 0.f;
    *reinterpret_cast<u32x4*>(gb + tok * hb + h0) =
        u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
  }
}

// ---------------------------------------------------------------- 1. dx (MFMA)

// k-steps per dx tile the MFMA kernel holds in registers.
template <int KS>
constexpr int dx_max_ksteps() { return KS >= 8 ? 25 : 32; }

// LDS: gamma[C] fp32, then W^T: row c holds W[0..ko)[c] (bf16; zero past n_out)
// with a pitch of 2*ko + 16 bytes.
// HDK = H*D/16 (H*D in {32, 64, 128}, q/k/v present, at most 16 bias heads):
// k-step j < 3 HDK reads q/k/v row `j / HDK` at a compile-time offset from one
// per-tile row pointer, and k-step 3 HDK (when there is a bias) the bias buffer.
template <int KS, int HDK>
__global__ __launch_bounds__(kThreads, 1) void bwd_dx_mfma(ProjProblem p, ProjBwdArgs a, const uint16_t* gb, int ko) {
  constexpr int C = 16 * KS;
  constexpr int CT = KS / 2;  // 32-channel tiles
  constexpr int NB = dx_max_ksteps<KS>();  // k-steps (16 outputs each) held in registers
  extern __shared__ __align__(16) char lds[];
  float* s_gamma = reinterpret_cast<float*>(lds);
  char* s_wt = lds + 4 * C;
  const int pw = 2 * ko + 16;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;

  {
    const uint16_t* wq = static_cast<const uint16_t*>(a.w_qkv);
    const uint16_t* wb = static_cast<const uint16_t*>(a.w_bias);
    constexpr int PIECES = C / 8;
    const int total = ko * PIECES;
    uint16_t* wt = reinterpret_cast<uint16_t*>(s_wt);
    const int pitch_e = pw / 2;
    for (int idx = tid; idx < total; idx += kThreads) {
      const int o = idx / PIECES;
      const int c8 = idx - o * PIECES;
      u32x4 w = {0, 0, 0, 0};
      if (o < p.n_qkv)
        w = reinterpret_cast<const u32x4*>(wq + static_cast<int64_t>(o) * C)[c8];
      else if (o < p.n_out)
        w = reinterpret_cast<const u32x4*>(wb + static_cast<int64_t>(o - p.n_qkv) * C)[c8];
      uint16_t* dst = wt + (8 * c8) * pitch_e + o;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[i * pitch_e] = static_cast<uint16_t>((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu));
    }
    for (int c = tid; c < C; c += kThreads) s_gamma[c] = a.gamma[c];
  }
  __syncthreads();

  const uint16_t* xg = static_cast<const uint16_t*>(a.x);
  uint16_t* dxg = static_cast<uint16_t*>(a.dx);
  constexpr float inv_c = 1.0f / C;
  const int stride = gridDim.x * kWaves;
  const int hb = bias_width(p);
  const uint16_t* const dqg = static_cast<const uint16_t*>(a.dq);
  const uint16_t* const dkg = static_cast<const uint16_t*>(a.dk);
  const uint16_t* const dvg = static_cast<const uint16_t*>(a.dv);

  // A tile's k-steps (q, k, v by 16-output steps, then the bias step) in two
  // register batches: batch 1 of a tile is requested, with its x and statistics, as
  // the tile starts; batch 0 of the next tile as soon as this tile's batch 0 has
  // been used.  So every batch's loads overlap half a tile's products (and the norm
  // backward), and the two batches together hold what one whole tile did.  Loads
  // are unconditional: a padding lane reads token 0 and its results are never stored.
  constexpr int NQ = 3 * HDK;
  constexpr int NK = NQ + 1;
  constexpr int N0 = (NK + 1) / 2, N1 = NK - N0;  // batch 1 ends with the bias step
  static_assert(HDK > 0 && NK <= NB, "q/k/v and bias k-steps must fit the register batches");
  const bool has_bias = hb > 0;
  auto token_of = [&](int tl) {
    const int64_t t = tile_token(p, tl, li);
    return t >= 0 ? t : int64_t{0};
  };
  auto load_step = [&](int j, int64_t tk, u32x4& g) {  // j is a compile-time constant after unrolling
    if (j < NQ) {
      const int w3 = j / HDK, c = j - (j / HDK) * HDK;
      const uint16_t* src = w3 == 0 ? dqg : (w3 == 1 ? dkg : dvg);
      g = *reinterpret_cast<const u32x4*>(src + tk * (16 * HDK) + 8 * half + 16 * c);
    } else {
      g = has_bias ? *reinterpret_cast<const u32x4*>(gb + tk * hb + 8 * half) : u32x4{0, 0, 0, 0};
    }
  };
  u32x4 g0[N0], g1[N1];
  auto load_batch0 = [&](int64_t tk) {
#pragma unroll
    for (int j = 0; j < N0; ++j) load_step(j, tk, g0[j]);
  };
  auto load_batch1 = [&](int64_t tk) {
#pragma unroll
    for (int j = 0; j < N1; ++j) load_step(N0 + j, tk, g1[j]);
  };
  // W^T operands of k-step ks for every channel tile.
  auto read_w = [&](int ks, u32x4* w) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      w[ct] = *reinterpret_cast<const u32x4*>(s_wt + (32 * ct + li) * pw + (16 * ks + 8 * half) * 2);
  };

  int tile = blockIdx.x * kWaves + wave;
  if (tile < p.tiles) load_batch0(token_of(tile));
  for (; tile < p.tiles; tile += stride) {
    const int64_t tok = tile_token(p, tile, li);
    const bool valid = tok >= 0;
    const int64_t tk = valid ? tok : 0;
    load_batch1(tk);
    // x at the accumulator's channels (32 ct + 8 g + 4 half + 0..3).
    u32x2 xr[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) xr[ct][g] = *reinterpret_cast<const u32x2*>(xg + tk * C + 32 * ct + 8 * g + 4 * half);
    const float mean = a.mean[tk];
    const float rstd = a.rstd[tk];

    // dy^T tile per 32 channels: D[c][t] = sum_o W^T[c][o] G[t][o].
    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};
    // Products of k-steps K0 .. K0 + n - 1: each step's W^T reads are issued one
    // step ahead, and a scheduling barrier keeps the compiler from hoisting more.
    auto run_steps = [&](auto k0_c, auto nmax_c, int n, const u32x4* g) {
      constexpr int K0 = decltype(k0_c)::value, NMAX = decltype(nmax_c)::value;
      u32x4 wc[CT], wn[CT];
      read_w(K0, wc);
#pragma unroll
      for (int j = 0; j < NMAX; ++j) {
        if (j < n) {
          if (j + 1 < n) read_w(K0 + j + 1, wn);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[ct] = mma(wc[ct], g[j], acc[ct]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) wc[ct] = wn[ct];
        }
      }
    };
    run_steps(std::integral_constant<int, 0>(), std::integral_constant<int, N0>(), N0, g0);
    if (tile + stride < p.tiles) load_batch0(token_of(tile + stride));
    run_steps(std::integral_constant<int, N0>(), std::integral_constant<int, N1>(), has_bias ? N1 : N1 - 1, g1);

    // Layer-norm backward on the token's channels (this lane's half, then the partner's).
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(s_gamma + 32 * ct + 8 * g + 4 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = xr[ct][g][e >> 1];
          const float xh = ((e & 1) ? hi_bf16(u) : lo_bf16(u)) - mean;
          const float gv = acc[ct][4 * g + e] * gm[e];
          acc[ct][4 * g + e] = gv;
          s1 += gv;
          s2 = fmaf(gv, xh * rstd, s2);
        }
      }
    s1 = pair_sum(s1) * inv_c;
    s2 = pair_sum(s2) * inv_c;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = xr[ct][g][e >> 1];
          const float xh = (((e & 1) ? hi_bf16(u) : lo_bf16(u)) - mean) * rstd;
          acc[ct][4 * g + e] = rstd * (acc[ct][4 * g + e] - s1 - xh * s2);
        }

    // Store: trade halves with the partner lane so each lane owns 8 consecutive
    // channels (low half: groups 1 and 3, high half: groups 0 and 2).
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
        const u32x4 out = {r0[0], r1[0], r0[1], r1[1]};
        if (valid) *reinterpret_cast<u32x4*>(dxg + tk * C + 32 * ct + 8 * (half ? g0 : g1)) = out;
      }
  }
}

// ---------------------------------------------------------------- 2. partial M, s (MFMA)

// LDS per stage: G [128 tokens][128 outputs] bf16 (pitch 288 B), then
// xhat [128 tokens][C] bf16 (pitch 2C + 32 B).  Two stages.
template <int KS>
constexpr int mpart_stage_bytes() { return kChunk * ((2 * kGroupOut + 32) + (32 * KS + 32)); }

template <int KS>
__global__ __launch_bounds__(kThreads, 1) void bwd_mpart_mfma(ProjProblem p, ProjBwdArgs a, const uint16_t* gb,
                                                             int n_groups, int ranges, int range_chunks, float* mpart,
                                                             float* spart) {
  constexpr int C = 16 * KS;
  constexpr int CT = KS / 2;
  constexpr int PG = 2 * kGroupOut + 32;
  constexpr int PX = 2 * C + 32;
  constexpr int STAGE = mpart_stage_bytes<KS>();
  constexpr int GPL = kGroupOut / 8;                 // G pieces per token
  constexpr int NGP = kChunk * GPL / kThreads;       // G pieces per thread
  constexpr int XPL = C / 8;                         // x pieces per token
  constexpr int XP = kChunk * XPL;
  constexpr int NXP = (XP + kThreads - 1) / kThreads;
  static_assert(kChunk * GPL % kThreads == 0, "G pieces must divide evenly");
  extern __shared__ __align__(16) char lds[];
  const uint32_t lds0 = lds_addr(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int n_ot = (p.n_out + 31) >> 5;
  const int blk = xcd_logical_block(blockIdx.x, n_groups * ranges);
  const int group = blk % n_groups;
  const int range = blk / n_groups;
  const int ot0 = 4 * group;
  const int n_ot_g = min(4, n_ot - ot0);
  const int ntile = n_ot_g * CT;
  const int64_t t_begin = static_cast<int64_t>(range) * range_chunks * kChunk;
  const int64_t t_end = min(p.T, t_begin + static_cast<int64_t>(range_chunks) * kChunk);
  const int nch = static_cast<int>((t_end - t_begin + kChunk - 1) / kChunk);
  const uint16_t* xg = static_cast<const uint16_t*>(a.x);

  // Every G piece of this thread has the same 8 outputs (kThreads is a multiple
  // of GPL): one source for the whole kernel.
  static_assert(kThreads % GPL == 0, "a thread's G pieces must share their outputs");
  const GSource gsrc = g_source(p, a, gb, 32 * ot0 + 8 * (tid % GPL));
  // One chunk's share of this thread in registers; two sets alternate so that a
  // chunk's loads are issued two chunks before its LDS stage is written.
  struct Regs {
    u32x4 g[NGP];
    u32x4 x[NXP];
    float m[NXP], r[NXP];
  };
  // Tokens past the range are loaded from its last token (no branch around the
  // loads) and staged as zeros.  The store also adds the staged G values to this
  // thread's column sums (its 8 outputs, summed over its tokens in order).
  auto load = [&](int ch, Regs& R) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ch) * kChunk;
#pragma unroll
    for (int i = 0; i < NGP; ++i) {
      const int64_t tok = min(t0 + (tid + i * kThreads) / GPL, t_end - 1);
      R.g[i] = g_load(gsrc, tok);
    }
#pragma unroll
    for (int i = 0; i < NXP; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / XPL;
      const int j = idx - t * XPL;
      const int64_t tok = min(t0 + t, t_end - 1);
      if (XP % kThreads == 0 || idx < XP) {
        R.x[i] = *reinterpret_cast<const u32x4*>(xg + tok * C + 8 * j);
        R.m[i] = a.mean[tok];
        R.r[i] = a.rstd[tok];
      }
    }
  };
  float s_part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto store = [&](const Regs& R, int ch, int buf) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ch) * kChunk;
    char* sg = lds + buf * STAGE;
    char* sx = sg + kChunk * PG;
#pragma unroll
    for (int i = 0; i < NGP; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / GPL;
      const int j = idx - t * GPL;
      const u32x4 gv = (gsrc.ok && t0 + t < t_end) ? R.g[i] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(sg + t * PG + 16 * j) = gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_part[2 * e] += lo_bf16(gv[e]);
        s_part[2 * e + 1] += hi_bf16(gv[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < NXP; ++i) {
      const int idx = tid + i * kThreads;
      if (XP % kThreads == 0 || idx < XP) {
        const int t = idx / XPL;
        const int j = idx - t * XPL;
        const bool in = t0 + t < t_end;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = in ? pack_bf16((lo_bf16(R.x[i][e]) - R.m[i]) * R.r[i], (hi_bf16(R.x[i][e]) - R.m[i]) * R.r[i]) : 0u;
        *reinterpret_cast<u32x4*>(sx + t * PX + 16 * j) = o;
      }
    }
  };
  // Transposed read: lane gets column col0 + lane % 32 at tokens 16 kk + 4 half + 0..3
  // and 16 kk + 8 + 4 half + 0..3 (the same token order for both operands).
  const int i16 = lane & 15;
  const int tr_row = 4 * half + (i16 >> 2);
  const int tr_col = (lane & 16) + 4 * (i16 & 3);
  auto tr = [&](uint32_t base, int pitch, int col0, int kk) {
    const uint32_t ad = base + (16 * kk + tr_row) * pitch + (col0 + tr_col) * 2;
    const u32x2 lo = lds_load_tr(ad);
    const u32x2 hi = lds_load_tr(ad + 8 * pitch);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // The wave's two product tiles wave and wave + kWaves; a tile past the group's
  // last (in a group of fewer than four output tiles) repeats the last one and is
  // not stored, so the loop has no branches.
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  int t_ot[2], t_ct[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tl = min(wave + kWaves * tt, ntile - 1);
    t_ot[tt] = tl / CT;
    t_ct[tt] = tl - t_ot[tt] * CT;
  }
  auto compute = [&](int buf) {
    const uint32_t sg = lds0 + buf * STAGE;
    const uint32_t sx = sg + kChunk * PG;
#pragma unroll 2
    for (int kk = 0; kk < kChunk / 16; ++kk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        acc[tt] = mma(tr(sg, PG, 32 * t_ot[tt], kk), tr(sx, PX, 32 * t_ct[tt], kk), acc[tt]);
  };

  // Chunk ch is staged in LDS buffer ch % 2; register set A carries even chunks,
  // B odd ones.
  Regs RA, RB;
  load(0, RA);
  if (nch > 1) load(1, RB);
  store(RA, 0, 0);
  __syncthreads();
  for (int ch = 0; ch < nch; ch += 2) {
    compute(0);
    if (ch + 2 < nch) load(ch + 2, RA);
    if (ch + 1 < nch) store(RB, ch + 1, 1);
    __syncthreads();
    if (ch + 1 >= nch) break;
    compute(1);
    if (ch + 3 < nch) load(ch + 3, RB);
    if (ch + 2 < nch) store(RA, ch + 2, 0);
    __syncthreads();
  }

  // D[o][c]: lane holds c = 32 ct + lane % 32, rows o = 32 ot + 8 (v/4) + 4 half + v % 4.
  const int po = padded_outputs(p);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tl = wave + kWaves * tt;
    if (tl < ntile) {
      const int ot = tl / CT, ct = tl - (tl / CT) * CT;
      float* dst = mpart + (static_cast<int64_t>(range) * po + 32 * (ot0 + ot)) * C + 32 * ct + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[static_cast<int64_t>(acc_row(v, lane)) * C] = acc[tt][v];
    }
  }
  // Column sums: thread tid holds outputs 8 (tid % GPL) + 0..7 of the group; the
  // kThreads / GPL threads of each output set are added in increasing order.
  constexpr int NSET = kThreads / GPL;
  float* sred = reinterpret_cast<float*>(lds);  // [NSET][kGroupOut], the stages are free
#pragma unroll
  for (int e = 0; e < 8; ++e) sred[(tid / GPL) * kGroupOut + 8 * (tid % GPL) + e] = s_part[e];
  __syncthreads();
  if (tid < 32 * n_ot_g) {
    float sum = 0.f;
    for (int m = 0; m < NSET; ++m) sum += sred[m * kGroupOut + tid];
    spart[static_cast<int64_t>(range) * po + 32 * ot0 + tid] = sum;
  }
}

// ---------------------------------------------------------------- vector kernels

constexpr int kVecTokens = 8;
constexpr int kVecThreads = 256;

template <typename T>
__device__ __forceinline__ float g_elem(const ProjProblem& p, const ProjBwdArgs& a, int64_t tok, int o) {
  if (o < p.n_qkv) {
    const int hd = p.H * p.D;
    const int which = o / hd;
    const T* src = static_cast<const T*>(which == 0 ? a.dq : (which == 1 ? a.dk : a.dv));
    return Elem<T>::load(src, tok * hd + (o - which * hd));
  }
  return a.dbias[bias_offset(p, o - p.n_qkv, tok)];
}

template <typename T>
__device__ __forceinline__ float w_elem(const ProjProblem& p, const ProjBwdArgs& a, int o, int c) {
  return o < p.n_qkv ? Elem<T>::load(static_cast<const T*>(a.w_qkv), static_cast<int64_t>(o) * p.C + c)
                     : Elem<T>::load(static_cast<const T*>(a.w_bias), static_cast<int64_t>(o - p.n_qkv) * p.C + c);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// dx for 8 tokens per workgroup: dy in LDS, then one wave per token.
template <typename T>
__global__ __launch_bounds__(kVecThreads) void bwd_dx_vector(ProjProblem p, ProjBwdArgs a) {
  extern __shared__ float dys[];  // [kVecTokens][C]
  const int C = p.C;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kVecTokens;
  for (int idx = threadIdx.x; idx < kVecTokens * C; idx += kVecThreads) {
    const int ti = idx / C;
    const int c = idx - ti * C;
    const int64_t tok = t0 + ti;
    float acc = 0.f;
    if (tok < p.T)
      for (int o = 0; o < p.n_out; ++o) acc = fmaf(g_elem<T>(p, a, tok, o), w_elem<T>(p, a, o, c), acc);
    dys[idx] = acc * a.gamma[c];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const T* x = static_cast<const T*>(a.x);
  for (int ti = threadIdx.x >> 6; ti < kVecTokens; ti += kVecThreads / 64) {
    const int64_t tok = t0 + ti;
    if (tok >= p.T) continue;
    const float mean = a.mean[tok], rstd = a.rstd[tok];
    float s1 = 0.f, s2 = 0.f;
    for (int c = lane; c < C; c += 64) {
      const float g = dys[ti * C + c];
      s1 += g;
      s2 = fmaf(g, (Elem<T>::load(x, tok * C + c) - mean) * rstd, s2);
    }
    s1 = wave_sum(s1) / C;
    s2 = wave_sum(s2) / C;
    for (int c = lane; c < C; c += 64) {
      const float xh = (Elem<T>::load(x, tok * C + c) - mean) * rstd;
      Elem<T>::store(static_cast<T*>(a.dx), tok * C + c, rstd * (dys[ti * C + c] - s1 - xh * s2));
    }
  }
}

// Partial M and s of one (range, output) pair per workgroup; threads over channels.
template <typename T>
__global__ __launch_bounds__(kVecThreads) void bwd_mpart_vector(ProjProblem p, ProjBwdArgs a, int range_tokens,
                                                                 float* mpart, float* spart) {
  const int o = blockIdx.x;
  const int range = blockIdx.y;
  const int64_t t_begin = static_cast<int64_t>(range) * range_tokens;
  const int64_t t_end = min(p.T, t_begin + range_tokens);
  const int po = padded_outputs(p);
  const T* x = static_cast<const T*>(a.x);
  for (int c = threadIdx.x; c < p.C; c += kVecThreads) {
    float m = 0.f, s = 0.f;
    for (int64_t t = t_begin; t < t_end; ++t) {
      const float g = g_elem<T>(p, a, t, o);
      m = fmaf(g, (Elem<T>::load(x, t * p.C + c) - a.mean[t]) * a.rstd[t], m);
      s += g;
    }
    mpart[(static_cast<int64_t>(range) * po + o) * p.C + c] = m;
    if (c == 0) spart[static_cast<int64_t>(range) * po + o] = s;
  }
}

// ---------------------------------------------------------------- 3. finalize

// One workgroup per output row o: M and s from the partials, dW, and the
// per-(o, c) products whose sums over o are dgamma and dbeta.  1024 threads = 8
// slots x 128 channels: slot k sums ranges k, k + 8, ... in increasing order (all
// its loads in flight at once), then the 8 slot sums are added in slot order.
constexpr int kFinSlots = 8;
constexpr int kFinCols = 128;
constexpr int kFinRowThreads = kFinSlots * kFinCols;

template <typename T>
__global__ __launch_bounds__(kFinRowThreads) void bwd_finalize_rows(ProjProblem p, ProjBwdArgs a, int ranges,
                                                                   const float* mpart, const float* spart,
                                                                   float* tgamma, float* tbeta) {
  __shared__ float part[kFinSlots][kFinCols];
  __shared__ float s_r[kFinRowThreads];
  __shared__ float s_sh;
  const int o = blockIdx.x;
  const int po = padded_outputs(p);
  const int slot = threadIdx.x / kFinCols;
  const int cl = threadIdx.x - slot * kFinCols;
  // s: every range's partial loaded at once, then summed in increasing range order.
  for (int r = threadIdx.x; r < ranges; r += kFinRowThreads) s_r[r] = spart[static_cast<int64_t>(r) * po + o];
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int r = 0; r < ranges; ++r) s += s_r[r];
    s_sh = s;
  }
  for (int c0 = 0; c0 < p.C; c0 += kFinCols) {
    const int c = c0 + cl;
    float m = 0.f;
    if (c < p.C) {
      const float* src = mpart + static_cast<int64_t>(o) * p.C + c;
      const int64_t rstride = static_cast<int64_t>(po) * p.C;
#pragma unroll 8
      for (int r = slot; r < ranges; r += kFinSlots) m += src[r * rstride];
    }
    part[slot][cl] = m;
    __syncthreads();
    if (slot == 0 && c < p.C) {
      m = part[0][cl];
#pragma unroll
      for (int k = 1; k < kFinSlots; ++k) m += part[k][cl];
      const float s = s_sh;
      const float dw = fmaf(m, a.gamma[c], s * a.beta[c]);
      if (o < p.n_qkv)
        a.dw_qkv[static_cast<int64_t>(o) * p.C + c] = dw;
      else
        a.dw_bias[static_cast<int64_t>(o - p.n_qkv) * p.C + c] = dw;
      const float w = w_elem<T>(p, a, o, c);
      tgamma[static_cast<int64_t>(o) * p.C + c] = w * m;
      tbeta[static_cast<int64_t>(o) * p.C + c] = w * s;
    }
    __syncthreads();
  }
}

// One workgroup per channel: thread i sums outputs i, i + 256, ... in order, then
// a fixed pairwise tree over the 256 partial sums.
__global__ __launch_bounds__(kVecThreads) void bwd_finalize_cols(ProjProblem p, ProjBwdArgs a, const float* tgamma,
                                                                 const float* tbeta) {
  __shared__ float sg[kVecThreads], sb[kVecThreads];
  const int c = blockIdx.x;
  float g = 0.f, b = 0.f;
  for (int o = threadIdx.x; o < p.n_out; o += kVecThreads) {
    g += tgamma[static_cast<int64_t>(o) * p.C + c];
    b += tbeta[static_cast<int64_t>(o) * p.C + c];
  }
  sg[threadIdx.x] = g;
  sb[threadIdx.x] = b;
  __syncthreads();
  for (int w = kVecThreads / 2; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) {
      sg[threadIdx.x] += sg[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.dgamma[c] = sg[0];
    a.dbeta[c] = sb[0];
  }
}

// ---------------------------------------------------------------- launch

bool use_mfma(const ProjProblem& p) { return p.dtype == 1 && (p.C == 32 || p.C == 64 || p.C == 128); }

// Outputs the dx kernel contracts over: q/k/v rows, then the bias buffer's
// columns, rounded up to whole 16-output k-steps.
int dx_ko(const ProjProblem& p) { return (p.n_qkv + bias_width(p) + 15) / 16 * 16; }

size_t dx_lds_bytes(const ProjProblem& p) {
  return static_cast<size_t>(4) * p.C + static_cast<size_t>(p.C) * (2 * dx_ko(p) + 16);
}

struct WsLayout {
  int ranges, range_chunks;
  size_t mpart, spart, tgamma, tbeta, gb, total;  // byte offsets
};

WsLayout ws_layout(const ProjProblem& p) {
  WsLayout w{};
  range_split(p, &w.ranges, &w.range_chunks);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t po = static_cast<size_t>(padded_outputs(p));
  w.mpart = 0;
  w.spart = up(w.mpart + static_cast<size_t>(w.ranges) * po * p.C * sizeof(float));
  w.tgamma = up(w.spart + static_cast<size_t>(w.ranges) * po * sizeof(float));
  w.tbeta = up(w.tgamma + static_cast<size_t>(p.n_out) * p.C * sizeof(float));
  w.gb = up(w.tbeta + static_cast<size_t>(p.n_out) * p.C * sizeof(float));
  w.total = up(w.gb + static_cast<size_t>(p.T) * bias_width(p) * sizeof(uint16_t));
  return w;
}

template <typename K>
hipError_t persistent_grid(K kern, size_t lds, int want, int* grid) {
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

// The dx kernels: MFMA when q/k/v rows are 32, 64 or 128 wide (and at most 16
// bias heads, and the weights fit in LDS), else the vector kernel.
bool dx_mfma_shape(const ProjProblem& p) {
  const int hd = p.H * p.D;
  return p.dtype == 1 && (p.C == 32 || p.C == 64 || p.C == 128) && p.n_qkv > 0 && bias_width(p) <= 16 &&
         (hd == 32 || hd == 64 || hd == 128) && dx_lds_bytes(p) <= kMaxLds;
}

hipError_t launch_dx_vector(const ProjProblem& p, const ProjBwdArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kVecTokens) * p.C * sizeof(float);
  const int64_t grid = (p.T + kVecTokens - 1) / kVecTokens;
  KernelTimer timer("ln_proj_bwd_dx_vector", s);
  if (p.dtype == 1)
    hipLaunchKernelGGL(bwd_dx_vector<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
  else
    hipLaunchKernelGGL(bwd_dx_vector<float>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
  return hipGetLastError();
}

template <int KS>
hipError_t launch_dx(const ProjProblem& p, const ProjBwdArgs& a, const uint16_t* gb, hipStream_t s) {
  if (!dx_mfma_shape(p)) return launch_dx_vector(p, a, s);
  const size_t lds = dx_lds_bytes(p);
  const int hd = p.H * p.D;
  auto kern = hd == 32 ? bwd_dx_mfma<KS, 2> : (hd == 64 ? bwd_dx_mfma<KS, 4> : bwd_dx_mfma<KS, 8>);
  int grid = 0;
  hipError_t e = persistent_grid(kern, lds, (p.tiles + kWaves - 1) / kWaves, &grid);
  if (e != hipSuccess) return e;
  KernelTimer timer("ln_proj_bwd_dx", s);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, p, a, gb, dx_ko(p));
  return hipGetLastError();
}

template <int KS>
hipError_t launch_mfma(const ProjProblem& p, const ProjBwdArgs& a, const WsLayout& w, char* ws, hipStream_t s) {
  hipError_t e;
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(ws + w.gb);
  if (bias_width(p) > 0) {
    KernelTimer timer("ln_proj_bwd_bias_tokens", s);
    hipLaunchKernelGGL(bias_grad_tokens, dim3(static_cast<unsigned>((p.T + 255) / 256)), dim3(256), 0, s, p, a,
                       reinterpret_cast<uint16_t*>(ws + w.gb));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_dx<KS>(p, a, gb, s)) != hipSuccess) return e;
  {
    const size_t lds = 2 * static_cast<size_t>(mpart_stage_bytes<KS>());
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_mpart_mfma<KS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int n_groups = ((p.n_out + 31) / 32 + 3) / 4;
    KernelTimer timer("ln_proj_bwd_mpart", s);
    hipLaunchKernelGGL(bwd_mpart_mfma<KS>, dim3(n_groups * w.ranges), dim3(kThreads), lds, s, p, a, gb, n_groups,
                       w.ranges, w.range_chunks, reinterpret_cast<float*>(ws + w.mpart),
                       reinterpret_cast<float*>(ws + w.spart));
    return hipGetLastError();
  }
}

}  // namespace

size_t ln_proj_bwd_workspace_bytes(const ProjProblem& p) { return ws_layout(p).total; }

hipError_t launch_ln_proj_bwd(const ProjProblem& p, const ProjBwdArgs& a, void* ws_ptr, hipStream_t s) {
  const WsLayout w = ws_layout(p);
  char* ws = static_cast<char*>(ws_ptr);
  float* mpart = reinterpret_cast<float*>(ws + w.mpart);
  float* spart = reinterpret_cast<float*>(ws + w.spart);
  float* tgamma = reinterpret_cast<float*>(ws + w.tgamma);
  float* tbeta = reinterpret_cast<float*>(ws + w.tbeta);
  hipError_t e = hipSuccess;
  const bool mf = use_mfma(p);
  if (mf) {
    switch (p.C) {
      case 32: e = launch_mfma<2>(p, a, w, ws, s); break;
      case 64: e = launch_mfma<4>(p, a, w, ws, s); break;
      default: e = launch_mfma<8>(p, a, w, ws, s); break;
    }
  } else {
    const int range_tokens = w.range_chunks * kChunk;
    if ((e = launch_dx_vector(p, a, s)) != hipSuccess) return e;
    KernelTimer timer("ln_proj_bwd_mpart_vector", s);
    if (p.dtype == 1)
      hipLaunchKernelGGL(bwd_mpart_vector<uint16_t>, dim3(p.n_out, w.ranges), dim3(kVecThreads), 0, s, p, a,
                         range_tokens, mpart, spart);
    else
      hipLaunchKernelGGL(bwd_mpart_vector<float>, dim3(p.n_out, w.ranges), dim3(kVecThreads), 0, s, p, a,
                         range_tokens, mpart, spart);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  {
    KernelTimer timer("ln_proj_bwd_finalize", s);
    if (p.dtype == 1)
      hipLaunchKernelGGL(bwd_finalize_rows<uint16_t>, dim3(p.n_out), dim3(kFinRowThreads), 0, s, p, a, w.ranges,
                         mpart, spart, tgamma, tbeta);
    else
      hipLaunchKernelGGL(bwd_finalize_rows<float>, dim3(p.n_out), dim3(kFinRowThreads), 0, s, p, a, w.ranges,
                         mpart, spart, tgamma, tbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finalize_cols, dim3(p.C), dim3(kVecThreads), 0, s, p, a, tgamma, tbeta);
  }
  return hipGetLastError();
}

}  // namespace evo
