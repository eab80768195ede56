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
//      32-output tiles, token range); G and xhat are staged in LDS per 64 tokens
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
constexpr int kChunk = 64;       // tokens per staged chunk of the partial-sum kernel
constexpr int kGroupOut = 128;   // outputs per group (four 32-output tiles)
constexpr int kMaxRanges = 64;   // token ranges of the partial sums
constexpr size_t kMaxLds = 160 * 1024;

// Rows of the partial-M array: outputs padded to whole 32-output tiles.
__host__ __device__ __forceinline__ int padded_outputs(const ProjProblem& p) { return (p.n_out + 31) / 32 * 32; }

// Number of token ranges and 64-token chunks per range.
void range_split(const ProjProblem& p, int* ranges, int* range_chunks) {
  const int64_t chunks = (p.T + kChunk - 1) / kChunk;
  int64_t r = chunks < kMaxRanges ? chunks : kMaxRanges;
  const int64_t per = (chunks + r - 1) / r;
  r = (chunks + per - 1) / per;  // every range holds at least one token
  *ranges = static_cast<int>(r);
  *range_chunks = static_cast<int>(per);
}

// 8 upstream gradients G[tok][o0 .. o0+7] as packed bf16 (o0 a multiple of 8):
// a 16-byte load of a dq/dk/dv row, or the bias heads gathered from dbias.
__device__ __forceinline__ u32x4 g_piece(const ProjProblem& p, const ProjBwdArgs& a, int64_t tok, int o0) {
  if (o0 >= p.n_out) return u32x4{0, 0, 0, 0};
  const int hd = p.H * p.D;
  if (o0 + 8 <= p.n_qkv) {
    const int which = o0 / hd;
    const int col = o0 - which * hd;
    const uint16_t* src = static_cast<const uint16_t*>(which == 0 ? a.dq : (which == 1 ? a.dk : a.dv));
    return *reinterpret_cast<const u32x4*>(src + tok * hd + col);
  }
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int o = o0 + e;
    v[e] = (o >= p.n_qkv && o < p.n_out) ? a.dbias[bias_offset(p, o - p.n_qkv, tok)] : 0.f;
  }
  return u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
}

// ---------------------------------------------------------------- 1. dx (MFMA)

// LDS: gamma[C] fp32, then W^T: row c holds W[0..ko)[c] (bf16; zero past n_out)
// with a pitch of 2*ko + 16 bytes.
template <int KS>
__global__ __launch_bounds__(kThreads, 1) void bwd_dx_mfma(ProjProblem p, ProjBwdArgs a, int ko) {
  constexpr int C = 16 * KS;
  constexpr int CT = KS / 2;  // 32-channel tiles
  constexpr int NB = KS >= 8 ? 4 : 8;  // k-steps (16 outputs each) per batch of G loads
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
  const int nks = ko / 16;
  const int nks_q = p.n_qkv / 16;  // k-steps made only of q/k/v outputs
  const int nbatch = (nks_q + NB - 1) / NB;
  const int hd = p.H * p.D;
  constexpr float inv_c = 1.0f / C;
  const int stride = gridDim.x * kWaves;

  for (int tile = blockIdx.x * kWaves + wave; tile < p.tiles; tile += stride) {
    const int64_t tok = tile_token(p, tile, li);
    const bool valid = tok >= 0;
    const int64_t tk = valid ? tok : 0;

    // Full q/k/v k-steps: 16-byte loads of dq/dk/dv rows, in batches of NB.
    auto load_batch = [&](int b, u32x4* dst) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int ks = NB * b + j;
        u32x4 v = {0, 0, 0, 0};
        if (valid && ks < nks_q) {
          const int o0 = 16 * ks + 8 * half;
          const int which = o0 / hd;
          const uint16_t* src = static_cast<const uint16_t*>(which == 0 ? a.dq : (which == 1 ? a.dk : a.dv));
          v = *reinterpret_cast<const u32x4*>(src + tk * hd + (o0 - which * hd));
        }
        dst[j] = v;
      }
    };
    u32x4 gcur[NB], gnext[NB];
    load_batch(0, gcur);

    // x at the accumulator's channels: 32 ct + 8 g + 4 half + 0..3.
    u32x2 xr[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        xr[ct][g] = valid ? *reinterpret_cast<const u32x2*>(xg + tk * C + 32 * ct + 8 * g + 4 * half)
                          : u32x2{0, 0};
    const float mean = valid ? a.mean[tk] : 0.f;
    const float rstd = valid ? a.rstd[tk] : 0.f;

    // dy^T tile per 32 channels: D[c][t] = sum_o W^T[c][o] G[t][o].
    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};
    auto step = [&](int ks, const u32x4& g) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(s_wt + (32 * ct + li) * pw + (16 * ks + 8 * half) * 2);
        acc[ct] = mma(w, g, acc[ct]);
      }
    };
    for (int b = 0; b < nbatch; ++b) {
      if (b + 1 < nbatch) load_batch(b + 1, gnext);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (NB * b + j < nks_q) step(NB * b + j, gcur[j]);
#pragma unroll
      for (int j = 0; j < NB; ++j) gcur[j] = gnext[j];
    }
    // Remaining k-steps: the pair-bias heads (and a last half q/k/v step).
    for (int ks = nks_q; ks < nks; ++ks) step(ks, valid ? g_piece(p, a, tk, 16 * ks + 8 * half) : u32x4{0, 0, 0, 0});

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

// LDS per stage: G [64 tokens][128 outputs] bf16 (pitch 288 B), then
// xhat [64 tokens][C] bf16 (pitch 2C + 32 B).  Two stages.
template <int KS>
constexpr int mpart_stage_bytes() { return kChunk * ((2 * kGroupOut + 32) + (32 * KS + 32)); }

template <int KS>
__global__ __launch_bounds__(kThreads, 1) void bwd_mpart_mfma(ProjProblem p, ProjBwdArgs a, int n_groups, int ranges,
                                                             int range_chunks, float* mpart, float* spart) {
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

  u32x4 gr[NGP];
  u32x4 xr[NXP];
  float xm[NXP], xs[NXP];
  auto load = [&](int ch) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ch) * kChunk;
#pragma unroll
    for (int i = 0; i < NGP; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / GPL;
      const int j = idx - t * GPL;
      const int64_t tok = t0 + t;
      gr[i] = tok < t_end ? g_piece(p, a, tok, 32 * ot0 + 8 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < NXP; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / XPL;
      const int j = idx - t * XPL;
      const int64_t tok = t0 + t;
      if (idx < XP && tok < t_end) {
        xr[i] = *reinterpret_cast<const u32x4*>(xg + tok * C + 8 * j);
        xm[i] = a.mean[tok];
        xs[i] = a.rstd[tok];
      } else {
        xr[i] = u32x4{0, 0, 0, 0};
        xm[i] = 0.f;
        xs[i] = 0.f;
      }
    }
  };
  auto store = [&](int buf) {
    char* sg = lds + buf * STAGE;
    char* sx = sg + kChunk * PG;
#pragma unroll
    for (int i = 0; i < NGP; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / GPL;
      const int j = idx - t * GPL;
      *reinterpret_cast<u32x4*>(sg + t * PG + 16 * j) = gr[i];
    }
#pragma unroll
    for (int i = 0; i < NXP; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < XP) {
        const int t = idx / XPL;
        const int j = idx - t * XPL;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16((lo_bf16(xr[i][e]) - xm[i]) * xs[i], (hi_bf16(xr[i][e]) - xm[i]) * xs[i]);
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

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  float s_acc = 0.f;
  load(0);
  store(0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nch) load(ch + 1);
    const uint32_t sg = lds0 + buf * STAGE;
    const uint32_t sx = sg + kChunk * PG;
    if (tid < 32 * n_ot_g) {
      const uint16_t* col = reinterpret_cast<const uint16_t*>(lds + buf * STAGE) + tid;
#pragma unroll 8
      for (int t = 0; t < kChunk; ++t) s_acc += bf16_to_f32(col[t * (PG / 2)]);
    }
#pragma unroll
    for (int kk = 0; kk < kChunk / 16; ++kk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tl = wave + kWaves * tt;
        if (tl < ntile) {
          const int ot = tl / CT, ct = tl - (tl / CT) * CT;
          acc[tt] = mma(tr(sg, PG, 32 * ot, kk), tr(sx, PX, 32 * ct, kk), acc[tt]);
        }
      }
    if (ch + 1 < nch) store(buf ^ 1);
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
  if (tid < 32 * n_ot_g) spart[static_cast<int64_t>(range) * po + 32 * ot0 + tid] = s_acc;
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

// One workgroup per output row o: M and s from the partials (increasing range),
// dW, and the per-(o, c) products whose sums over o are dgamma and dbeta.
template <typename T>
__global__ __launch_bounds__(kVecThreads) void bwd_finalize_rows(ProjProblem p, ProjBwdArgs a, int ranges,
                                                                 const float* mpart, const float* spart,
                                                                 float* tgamma, float* tbeta) {
  const int o = blockIdx.x;
  const int po = padded_outputs(p);
  float s = 0.f;
  for (int r = 0; r < ranges; ++r) s += spart[static_cast<int64_t>(r) * po + o];
  for (int c = threadIdx.x; c < p.C; c += kVecThreads) {
    float m = 0.f;
    for (int r = 0; r < ranges; ++r) m += mpart[(static_cast<int64_t>(r) * po + o) * p.C + c];
    const float dw = fmaf(m, a.gamma[c], s * a.beta[c]);
    if (o < p.n_qkv)
      a.dw_qkv[static_cast<int64_t>(o) * p.C + c] = dw;
    else
      a.dw_bias[static_cast<int64_t>(o - p.n_qkv) * p.C + c] = dw;
    const float w = w_elem<T>(p, a, o, c);
    tgamma[static_cast<int64_t>(o) * p.C + c] = w * m;
    tbeta[static_cast<int64_t>(o) * p.C + c] = w * s;
  }
}

__global__ __launch_bounds__(kVecThreads) void bwd_finalize_cols(ProjProblem p, ProjBwdArgs a, const float* tgamma,
                                                                 const float* tbeta) {
  const int c = blockIdx.x * kVecThreads + threadIdx.x;
  if (c >= p.C) return;
  float g = 0.f, b = 0.f;
  for (int o = 0; o < p.n_out; ++o) {
    g += tgamma[static_cast<int64_t>(o) * p.C + c];
    b += tbeta[static_cast<int64_t>(o) * p.C + c];
  }
  a.dgamma[c] = g;
  a.dbeta[c] = b;
}

// ---------------------------------------------------------------- launch

bool use_mfma(const ProjProblem& p) { return p.dtype == 1 && (p.C == 32 || p.C == 64 || p.C == 128); }

int dx_ko(const ProjProblem& p) { return (p.n_out + 15) / 16 * 16; }

size_t dx_lds_bytes(const ProjProblem& p) {
  return static_cast<size_t>(4) * p.C + static_cast<size_t>(p.C) * (2 * dx_ko(p) + 16);
}

struct WsLayout {
  int ranges, range_chunks;
  size_t mpart, spart, tgamma, tbeta, total;  // byte offsets
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
  w.total = up(w.tbeta + static_cast<size_t>(p.n_out) * p.C * sizeof(float));
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

template <int KS>
hipError_t launch_mfma(const ProjProblem& p, const ProjBwdArgs& a, const WsLayout& w, char* ws, hipStream_t s) {
  hipError_t e;
  {
    const size_t lds = dx_lds_bytes(p);
    int grid = 0;
    if ((e = persistent_grid(bwd_dx_mfma<KS>, lds, (p.tiles + kWaves - 1) / kWaves, &grid)) != hipSuccess) return e;
    KernelTimer timer("ln_proj_bwd_dx", s);
    hipLaunchKernelGGL(bwd_dx_mfma<KS>, dim3(grid), dim3(kThreads), lds, s, p, a, dx_ko(p));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const size_t lds = 2 * static_cast<size_t>(mpart_stage_bytes<KS>());
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_mpart_mfma<KS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int n_groups = ((p.n_out + 31) / 32 + 3) / 4;
    KernelTimer timer("ln_proj_bwd_mpart", s);
    hipLaunchKernelGGL(bwd_mpart_mfma<KS>, dim3(n_groups * w.ranges), dim3(kThreads), lds, s, p, a, n_groups,
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
  const bool mf = use_mfma(p) && dx_lds_bytes(p) <= kMaxLds;
  if (mf) {
    switch (p.C) {
      case 32: e = launch_mfma<2>(p, a, w, ws, s); break;
      case 64: e = launch_mfma<4>(p, a, w, ws, s); break;
      default: e = launch_mfma<8>(p, a, w, ws, s); break;
    }
  } else {
    const size_t lds = static_cast<size_t>(kVecTokens) * p.C * sizeof(float);
    const int64_t grid = (p.T + kVecTokens - 1) / kVecTokens;
    const int range_tokens = w.range_chunks * kChunk;
    {
      KernelTimer timer("ln_proj_bwd_dx_vector", s);
      if (p.dtype == 1)
        hipLaunchKernelGGL(bwd_dx_vector<uint16_t>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
      else
        hipLaunchKernelGGL(bwd_dx_vector<float>, dim3(static_cast<unsigned>(grid)), dim3(kVecThreads), lds, s, p, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
      hipLaunchKernelGGL(bwd_finalize_rows<uint16_t>, dim3(p.n_out), dim3(kVecThreads), 0, s, p, a, w.ranges, mpart,
                         spart, tgamma, tbeta);
    else
      hipLaunchKernelGGL(bwd_finalize_rows<float>, dim3(p.n_out), dim3(kVecThreads), 0, s, p, a, w.ranges, mpart,
                         spart, tgamma, tbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_finalize_cols, dim3((p.C + kVecThreads - 1) / kVecThreads), dim3(kVecThreads), 0, s, p, a,
                       tgamma, tbeta);
  }
  return hipGetLastError();
}

}  // namespace evo
