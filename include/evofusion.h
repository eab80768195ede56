/*
 * evofusion.h -- C ABI of the fused layer norm + projections that produce the
 * inputs of EvoAttention (evoattn.h), in the same library (libevoattn.so).
 *
 * The operation (MegaFold, gist.science technical summary, Methodik section 3
 * "EvoFusion": layer normalisation and the linear projections after it are one
 * operator whose inner loops are restructured so that the normalised tensor is
 * never written to HBM between the two; the pages give no formulas, so this is
 * the textbook layer norm followed by bias-free projections).  For every token
 * t = (a, b) of x [A, B, C]:
 *
 *   mean[t] = (1/C) sum_c x[t,c]
 *   rstd[t] = 1 / sqrt((1/C) sum_c (x[t,c] - mean[t])^2 + eps)   (biased variance)
 *   y[t,c]  = (x[t,c] - mean[t]) * rstd[t] * gamma[c] + beta[c]
 *   q[a,b,h,e] = sum_c y[t,c] w_qkv[h*d + e, c]
 *   k[a,b,h,e] = sum_c y[t,c] w_qkv[H*d + h*d + e, c]
 *   v[a,b,h,e] = sum_c y[t,c] w_qkv[2*H*d + h*d + e, c]
 *   bias[h,a,b] = sum_c y[(a,b),c] w_bias[h,c]     bias_transpose == 0
 *   bias[h,a,b] = sum_c y[(b,a),c] w_bias[h,c]     bias_transpose == 1
 *
 * q, k, v keep x's token order: for a pair tensor z [N, N, C] they are the
 * attention's [R, N, H, d] inputs for the starting node (transpose = 0 in
 * evoattn_fwd) and its [N, R, H, d] inputs for the ending node (transpose = 1).
 * The bias is [H, N, N] in the attention's kernel frame: bias_transpose = 0 for
 * the starting node, 1 for the ending node (whose query is the pair tensor's
 * column index).  For MSA row attention, project the MSA tensor with w_bias =
 * NULL and the pair tensor with w_qkv = NULL.
 *
 * ---------------------------------------------------------------- layouts
 * Dense, row-major.  x [A][B][C]; w_qkv [3*H*d][C] (the layout of a torch
 * Linear weight); w_bias [H][C]; q, k, v [A][B][H][d]; bias [H][A][B];
 * gamma, beta [C] fp32; mean, rstd [A*B] fp32.
 * dtype EVOATTN_BF16: x, w_qkv, w_bias, q, k, v, bias are bfloat16; the
 *   statistics and every sum are fp32, and y is rounded to bf16 before the
 *   projections (what an unfused bf16 pipeline stores between the two).
 * dtype EVOATTN_FP32: the same arrays are float.
 *
 * ---------------------------------------------------------------- ownership
 * Every pointer except `stream` is a device pointer owned by the caller.  The
 * library allocates nothing; outputs are overwritten; inputs and outputs must
 * not overlap.  The backward's scratch space is passed in as `workspace` of at
 * least evoattn_ln_proj_bwd_workspace_bytes() (256-byte aligned; contents on
 * entry do not matter).  Work is enqueued on `stream` (NULL = default stream).
 *
 * ---------------------------------------------------------------- errors
 * Arguments are validated before anything is enqueued; the return value is an
 * evoattn_status_t and evoattn_last_error_detail() describes a failure.
 *
 * Supported: A, B, H >= 1; d in {8, 16, 32, 64}; 16 <= C <= 2048 with C a
 * multiple of 8; A*B < 2^31 and A*B*max(C, 3*H*d) < 2^31 elements; with
 * w_bias, A == B.  Pointers 16-byte aligned (gamma, beta, mean, rstd: 4).
 * The bf16 MFMA kernel covers C in {32, 64, 128} when the weights fit in
 * LDS; other shapes run a vector-ALU kernel with the same results.
 */
#ifndef EVOFUSION_H
#define EVOFUSION_H

#include "evoattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Forward.  w_qkv and w_bias may each be NULL (not both); q, k, v must be
 * non-NULL exactly when w_qkv is, bias exactly when w_bias is.  mean and rstd
 * (both or neither) receive the per-token statistics the backward needs. */
evoattn_status_t evoattn_ln_proj_fwd(int64_t a, int64_t b, int64_t channels, int64_t heads,
                                     int64_t head_dim, int dtype, int bias_transpose, float eps,
                                     const void* x, const float* gamma, const float* beta,
                                     const void* w_qkv, const void* w_bias,
                                     void* q, void* k, void* v, void* bias,
                                     float* mean, float* rstd, void* stream);

/* Bytes of workspace evoattn_ln_proj_bwd needs (fixed-order partial sums over
 * at most 64 token ranges; O((3*H*d + H) * C)).  with_qkv / with_bias say which
 * weights the call has.  Returns 0 and records an error detail if the problem
 * is invalid. */
size_t evoattn_ln_proj_bwd_workspace_bytes(int64_t a, int64_t b, int64_t channels, int64_t heads,
                                           int64_t head_dim, int dtype, int with_qkv, int with_bias);

/* Backward of L = sum q*dq + sum k*dk + sum v*dv + sum bias*dbias through the
 * forward above.  Inputs: the forward's x, gamma, beta, weights, its mean and
 * rstd (required), and the upstream gradients dq, dk, dv (dtype, layout of q;
 * exactly when w_qkv is given) and dbias (fp32 [H, A, B] in the kernel frame
 * as evoattn_bwd writes it; exactly when w_bias is given).  Outputs: dx (dtype,
 * layout of x), dgamma, dbeta (fp32 [C]), dw_qkv (fp32 [3*H*d, C], with w_qkv)
 * and dw_bias (fp32 [H, C], with w_bias).  The sums over tokens run in a fixed
 * order: results are bit-identical across calls with the same inputs.  In bf16
 * mode dbias and xhat are rounded to bf16 as matrix-core operands; every sum is
 * fp32. */
evoattn_status_t evoattn_ln_proj_bwd(int64_t a, int64_t b, int64_t channels, int64_t heads,
                                     int64_t head_dim, int dtype, int bias_transpose,
                                     const void* x, const float* gamma, const float* beta,
                                     const void* w_qkv, const void* w_bias,
                                     const float* mean, const float* rstd,
                                     const void* dq, const void* dk, const void* dv, const float* dbias,
                                     void* dx, float* dgamma, float* dbeta, float* dw_qkv, float* dw_bias,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- transition
 * The SwiGLU transition of a pair or MSA tensor (MegaFold, gist.science
 * technical summary, Methodik section 3 "EvoFusion": SwiGLU is one of the fused
 * operators; no formula is printed, this is the plainest reading).  For every
 * token t of x [A, B, C], with y the layer norm above (biased variance, eps in
 * the square root, per-channel gamma and beta):
 *
 *   a[t,j] = sum_c y[t,c] w_a[j,c],   b[t,j] = sum_c y[t,c] w_b[j,c]   (j < n*C)
 *   h[t,j] = silu(a[t,j]) * b[t,j],   silu(z) = z / (1 + exp(-z))
 *   out[t,c] = sum_j h[t,j] w_out[c,j]
 *
 * Layouts: x, out [A][B][C]; w_a, w_b [n*C][C]; w_out [C][n*C] (torch Linear
 * weights); gamma, beta [C] fp32; mean, rstd [A*B] fp32.  bf16 only (y and h are
 * rounded to bf16 as matrix-core operands; sums and statistics are fp32), C in
 * {64, 128}, expansion n in 1..16.  Other shapes return EVOATTN_ERR_UNSUPPORTED.
 * y, a, b and h are never written to memory. */
evoattn_status_t evoattn_transition_fwd(int64_t a, int64_t b, int64_t channels, int64_t expansion, int dtype,
                                        float eps, const void* x, const float* gamma, const float* beta,
                                        const void* w_a, const void* w_b, const void* w_out, void* out,
                                        float* mean, float* rstd, void* stream);

/* Bytes of workspace evoattn_transition_bwd needs (fixed-order partial sums of the
 * weight gradients over at most 64 token ranges: O(ranges * n*C * C), plus the
 * normalised input xhat in bf16, a*b*C*2 bytes, written by the dx pass and read by
 * the weight-gradient pass).  Returns 0 and records an error detail if the
 * problem is invalid or unsupported. */
size_t evoattn_transition_bwd_workspace_bytes(int64_t a, int64_t b, int64_t channels, int64_t expansion,
                                              int dtype);

/* Backward of L = sum out * dout through evoattn_transition_fwd.  Inputs: the
 * forward's inputs, its mean and rstd (required), dout (bf16, layout of x).
 * Outputs: dx (bf16), dgamma, dbeta (fp32 [C]), dw_a, dw_b (fp32 [n*C, C]),
 * dw_out (fp32 [C, n*C]).  a, b and h are recomputed on chip, never stored; the
 * sums over tokens run in a fixed order (bit-identical across calls).  da, db,
 * h, y and xhat are rounded to bf16 as matrix-core operands (the backward forms y
 * from the rounded xhat); sums are fp32. */
evoattn_status_t evoattn_transition_bwd(int64_t a, int64_t b, int64_t channels, int64_t expansion, int dtype,
                                        const void* x, const float* gamma, const float* beta,
                                        const void* w_a, const void* w_b, const void* w_out,
                                        const float* mean, const float* rstd, const void* dout,
                                        void* dx, float* dgamma, float* dbeta,
                                        float* dw_a, float* dw_b, float* dw_out,
                                        void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EVOFUSION_H */
