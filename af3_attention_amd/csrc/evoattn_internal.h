// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

// Problem description handed to every kernel launcher.  Element (r, p, h, c)
// of q/k/v/o/dout/dq/dk/dv lives at ((r*row_stride + p*pos_stride)*H + h)*D + c,
// so transpose only changes the two strides.
struct Problem {
  int R, N, H, D;
  int dtype;          // 0 fp32, 1 bf16
  int transpose;
  int64_t row_stride; // in positions: N when transpose == 0, 1 otherwise
  int64_t pos_stride; // in positions: 1 when transpose == 0, R otherwise
  float scale;        // 1/sqrt(D)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;   // [H,N,N] or nullptr
  const float* mask;  // [R,N] or nullptr
  void* o;
  float* lse;         // [R,H,N] or nullptr
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  const float* mask;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dbias;       // [H,N,N] or nullptr
  float* delta;       // workspace [R,H,N]: sum_c dout*o per softmax row
  void* qaug;         // MFMA path workspace [R,H,N] x 16 B: per-query split operands (lse, delta)
                      // for the dq and dkdv kernels, nullptr when they do not run
  void* kaug;         // MFMA path workspace [R,N] x 16 B: per-key split operands (mask)
  void* qops;         // MFMA path workspace [R,H,Np] x 32 B (Np = N rounded up to 128): per
                      // query the complete operands of the S and dP steps (fused, dbias)
  float* scratch;     // further workspace (path specific)
  size_t scratch_bytes;
};

// Brackets one kernel launch with HIP events on its stream while timing is
// enabled (evoattn_timing_enable); a no-op otherwise.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

// Vector-ALU path: any supported head_dim, fp32 or bf16 storage, fp32 math.
hipError_t launch_fwd_vector(const Problem& p, const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_vector(const Problem& p, const BwdArgs& a, hipStream_t s);

// bf16 MFMA path (gfx950 matrix cores), fp32 accumulation.  Workspace sizes in
// bytes; the launchers carve their scratch out of `ws`.
size_t fwd_mfma_workspace_bytes(const Problem& p);
size_t bwd_mfma_workspace_bytes(const Problem& p);
hipError_t launch_fwd_mfma(const Problem& p, const FwdArgs& a, void* ws, hipStream_t s);
hipError_t launch_bwd_mfma(const Problem& p, const BwdArgs& a, void* ws, hipStream_t s);

// dQ (kernels_bwd_dq.hip); bias_q is the query-lane tiled bias.
hipError_t launch_dq_pipe(const Problem& p, const BwdArgs& a, const float* bias_q, hipStream_t s);

// dK, dV (kernels_bwd_dkdv.hip); bias_k is the key-lane tiled bias.
hipError_t launch_dkdv_pipe(const Problem& p, const BwdArgs& a, const float* bias_k, hipStream_t s);

// dBias partial sums over fixed row groups (kernels_bwd_dbias.hip): out[g][h][j][k].
int dbias_pipe_groups(const Problem& p);
hipError_t launch_dbias_pipe(const Problem& p, const BwdArgs& a, const float* bias_k, int groups, float* out,
                             hipStream_t s);

// Layer norm + projections of a token tensor x [A, B, C] into the attention's
// inputs (kernels_ln_proj.hip).  Output row o < n_qkv goes to q (o < H*D), k
// or v at [token][o % (H*D)]; rows n_qkv <= o < n_out are the pair-bias heads.
struct ProjProblem {
  int A, B, C, H, D;
  int64_t T;           // tokens A*B
  int dtype;           // 0 fp32, 1 bf16
  int bias_transpose;  // bias[h][a][b] from token (b, a) instead of (a, b)
  int n_qkv;           // 3*H*D, or 0 without q/k/v
  int n_out;           // n_qkv + (H with bias, else 0)
  int col_tiles;       // 32-token tiles run down a column of the A x B grid
  int tiles;           // number of 32-token tiles
  float eps;
};

struct ProjFwdArgs {
  const void* x;
  const float* gamma;
  const float* beta;
  const void* w_qkv;   // [n_qkv][C] or nullptr
  const void* w_bias;  // [H][C] or nullptr
  void* q;
  void* k;
  void* v;
  void* bias;          // [H][A][B] or nullptr
  float* mean;         // [T] or nullptr
  float* rstd;         // [T] or nullptr
};

hipError_t launch_ln_proj_fwd(const ProjProblem& p, const ProjFwdArgs& a, hipStream_t s);

struct ProjBwdArgs {
  const void* x;
  const float* gamma;
  const float* beta;
  const void* w_qkv;   // [n_qkv][C] or nullptr
  const void* w_bias;  // [H][C] or nullptr
  const float* mean;   // [T]
  const float* rstd;   // [T]
  const void* dq;      // upstream gradients of q, k, v [T][H*D] (with w_qkv)
  const void* dk;
  const void* dv;
  const float* dbias;  // upstream gradient of the bias [H][A][B] fp32 (with w_bias)
  void* dx;            // [T][C]
  float* dgamma;       // [C]
  float* dbeta;        // [C]
  float* dw_qkv;       // [n_qkv][C] (with w_qkv)
  float* dw_bias;      // [H][C] (with w_bias)
};

// Workspace of the backward in bytes, and its launch.
size_t ln_proj_bwd_workspace_bytes(const ProjProblem& p);
hipError_t launch_ln_proj_bwd(const ProjProblem& p, const ProjBwdArgs& a, void* ws, hipStream_t s);

// SwiGLU transition of a token tensor x [A, B, C] (kernels_transition*.hip):
// out = (silu(y w_a^T) * (y w_b^T)) w_out^T with y the layer norm of x.
struct TransProblem {
  int A, B, C;
  int hidden;  // expansion * C
  int64_t T;   // tokens A*B
  int tiles;   // 32-token tiles
  float eps;
};

struct TransFwdArgs {
  const void* x;
  const float* gamma;
  const float* beta;
  const void* w_a;    // [hidden][C]
  const void* w_b;    // [hidden][C]
  const void* w_out;  // [C][hidden]
  void* out;          // [T][C]
  float* mean;        // [T] or nullptr
  float* rstd;        // [T] or nullptr
};

struct TransBwdArgs {
  const void* x;
  const float* gamma;
  const float* beta;
  const void* w_a;
  const void* w_b;
  const void* w_out;
  const float* mean;
  const float* rstd;
  const void* dout;   // [T][C]
  void* dx;           // [T][C]
  float* dgamma;      // [C]
  float* dbeta;       // [C]
  float* dw_a;        // [hidden][C]
  float* dw_b;        // [hidden][C]
  float* dw_out;      // [C][hidden]
};

hipError_t launch_transition_fwd(const TransProblem& p, const TransFwdArgs& a, hipStream_t s);
size_t transition_bwd_workspace_bytes(const TransProblem& p);
hipError_t launch_transition_bwd(const TransProblem& p, const TransBwdArgs& a, void* ws, hipStream_t s);

// bf16 storage conversions (round to nearest even; NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

}  // namespace evo
