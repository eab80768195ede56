/*
 * evoattn.h -- C ABI of the MI355X (gfx950) library for memory-efficient 3D
 * attention over a 2D pair representation with an additively broadcast pair
 * bias ("EvoAttention"), forward and backward.
 *
 * The operation (MegaFold, gist.science technical summary, Methodik section 1
 * "EvoFlash-3D"; the pages describe it in words only): for every attention row
 * r < R, head h < H and query position j < N,
 *
 *   o[r,j,h,:] = sum_k softmax_k( q[r,j,h,:].k[r,k,h,:] / sqrt(d)
 *                                 + bias[h,j,k] + mask[r,k] ) v[r,k,h,:]
 *
 * The bias is shared by all rows r.  Starting-node triangle attention has
 * R = N (rows of the pair tensor); MSA row attention has R = number of MSA
 * rows; ending-node triangle attention is the same operation on the transposed
 * pair layout (transpose = 1).  The pages' point is that the R*H*N*N logit
 * tensor is never stored: the library computes it tile by tile on chip with an
 * online softmax, in the forward and in the backward, so extra memory is
 * O(R*H*N + H*N*N).
 *
 * ---------------------------------------------------------------- layouts
 * All arrays are dense and row-major.  "Kernel frame" indices (r, p, h, c):
 *   q, k, v, o, dout, dq, dk, dv : element (r,p,h,c) lives at
 *        [r][p][h][c]   (physical shape [R, N, H, d]) when transpose == 0,
 *        [p][r][h][c]   (physical shape [N, R, H, d]) when transpose == 1.
 *   bias   : [H][N][N], bias[h][j][k]; query j, key k.  Always kernel frame
 *            (for the ending node pass the bias of the transposed pair).
 *   mask   : [R][N] fp32, additive, mask[r][k] for key k of row r; 0 or -inf
 *            (finite values are allowed; +inf and NaN are not).
 *   lse    : [R][H][N] fp32, natural-log logsumexp of each softmax row
 *            (r, h, j); -inf for a row whose keys are all masked.
 *   dbias  : [H][N][N] fp32, sum over rows r of dS[r,h,j,k], reduced in a
 *            fixed order: bit-identical across calls with the same inputs.
 *
 * dtype EVOATTN_FP32: q, k, v, bias, o, dout, dq, dk, dv are float.
 * dtype EVOATTN_BF16: the same arrays are bfloat16 (uint16 bit patterns),
 *   outputs rounded to nearest even; every accumulation is fp32.
 * mask, lse and dbias are fp32 in both modes.
 *
 * A row whose keys are all masked yields o = 0, lse = -inf and contributes
 * nothing to any gradient.
 *
 * ---------------------------------------------------------------- ownership
 * Every pointer argument except `stream` is a device pointer owned by the
 * caller.  The library allocates no device memory and keeps no state between
 * calls beyond a thread-local error string, the device address of
 * evoattn_fwd_noalloc's static scratch (one per device, looked up once) and,
 * while timing is enabled, the per-kernel timing record (see below).  Outputs are overwritten, never
 * accumulated.  Scratch space is passed in as `workspace` of at least the size
 * the matching *_workspace_bytes query returns; its contents on entry do not
 * matter and on return are unspecified.  Inputs and outputs must not overlap.
 *
 * ---------------------------------------------------------------- errors
 * Every entry point validates all arguments before it enqueues anything and
 * returns a status; no exception crosses this boundary.  Work is enqueued on
 * `stream` (a hipStream_t; NULL is the default stream) and runs
 * asynchronously; a fault during execution surfaces at the caller's next
 * synchronisation with that stream.  A launch that HIP rejects returns
 * EVOATTN_ERR_DEVICE.  evoattn_last_error_detail() describes the last failure
 * on the calling thread.
 *
 * Supported: R, N, H >= 1; d in {8, 16, 32, 64}; R*N*H*d < 2^31 elements per
 * q/k/v tensor and H*N*N < 2^31; pointers 16-byte aligned (mask, lse, dbias
 * 4-byte aligned).
 */
#ifndef EVOATTN_H
#define EVOATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EVOATTN_ABI_VERSION 1

typedef enum {
  EVOATTN_OK = 0,
  EVOATTN_ERR_INVALID_ARGUMENT = 1, /* null pointer, size < 1, misalignment, bad enum */
  EVOATTN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head_dim, size limits) */
  EVOATTN_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required */
  EVOATTN_ERR_DEVICE = 4            /* HIP reported an error (no device, launch failure) */
} evoattn_status_t;

typedef enum {
  EVOATTN_FP32 = 0,
  EVOATTN_BF16 = 1
} evoattn_dtype_t;

/* Returns EVOATTN_ABI_VERSION of the built library.  (Interface versioning of
 * this boundary; not part of the pages' method.) */
int evoattn_abi_version(void);

/* Static, never-NULL name of a status code.  (Error reporting of this boundary;
 * not part of the pages' method.) */
const char* evoattn_status_string(int status);

/* Description of the last failed call on the calling thread ("" if none).
 * (Error reporting of this boundary; not part of the pages' method.) */
const char* evoattn_last_error_detail(void);

/* Scratch of the tile-by-tile forward (gist.science MegaFold technical summary,
 * Methodik section 1: the logits stay on chip, so the scratch is O(R*N + H*N*N)).
 * Bytes of workspace evoattn_fwd needs for this problem (may be 0): for bf16
 * the sqrt(d)-scaled bias as fp32 tiles (O(H*N*N)) and, for head_dim <= 32, the
 * key-side mask operands and each row's last unmasked key (O(R*N)).
 * Returns 0 and records an error detail if the problem is invalid. */
size_t evoattn_fwd_workspace_bytes(int64_t rows, int64_t n, int64_t heads,
                                   int64_t head_dim, int dtype);

/* Scratch of the recomputing backward (same passage: the memory-efficient kernel
 * runs in the backward too).  Bytes of workspace evoattn_bwd needs for this
 * problem (row statistics, the tiled bias and the fixed-order dBias partial sums;
 * O(R*H*N + H*N*N)). */
size_t evoattn_bwd_workspace_bytes(int64_t rows, int64_t n, int64_t heads,
                                   int64_t head_dim, int dtype);

/* Forward of EvoAttention (gist.science MegaFold technical summary, Methodik
 * section 1 "EvoFlash-3D": the logits of each row are formed tile by tile on
 * chip and normalised with an online softmax; the pair bias is added to every
 * row).  Inputs q, k, v (dtype, layout above), bias [H,N,N] (dtype; NULL means
 * zero), mask [R,N] fp32 (NULL means zero).  Outputs o (dtype, same layout as
 * q) and lse [R,H,N] fp32 (NULL if no backward will follow). */
evoattn_status_t evoattn_fwd(int64_t rows, int64_t n, int64_t heads, int64_t head_dim,
                             int dtype, int transpose,
                             const void* q, const void* k, const void* v,
                             const void* bias, const float* mask,
                             void* o, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Forward without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as evoattn_fwd, minus the workspace:
 * the library uses a static device array of EVOATTN_NOALLOC_SCRATCH_BYTES per
 * device instead (held until the process ends; no hipMalloc/hipFree or other
 * allocating call is made).  Returns EVOATTN_ERR_WORKSPACE when the problem needs
 * more scratch than that (evoattn_fwd_workspace_bytes tells).  Every call on a
 * device shares that device's array: calls that overlap in time on one device
 * (different streams or threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs to start at zero. */
#define EVOATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
evoattn_status_t evoattn_fwd_noalloc(int64_t rows, int64_t n, int64_t heads, int64_t head_dim,
                                     int dtype, int transpose,
                                     const void* q, const void* k, const void* v,
                                     const void* bias, const float* mask,
                                     void* o, float* lse, void* stream);

/* Backward of EvoAttention (same passage: the memory-efficient kernel also runs
 * in the backward pass, recomputing the probabilities from lse on chip; dbias is
 * the sum over rows of the bias gradient, reduced in a fixed order).  Backward
 * of sum(o * dout).  Inputs: the forward's inputs, its outputs o and lse
 * (required), and dout (dtype, layout of o).  Outputs dq, dk, dv (dtype, layout
 * of q) and dbias [H,N,N] fp32 (NULL to skip).  The mask receives no gradient. */
evoattn_status_t evoattn_bwd(int64_t rows, int64_t n, int64_t heads, int64_t head_dim,
                             int dtype, int transpose,
                             const void* q, const void* k, const void* v,
                             const void* bias, const float* mask,
                             const void* o, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv, float* dbias,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- timing
 * Per-kernel timing, a profiling aid (the measurement of the path, not part of
 * the pages' method).  While enabled, every kernel this
 * library launches is bracketed by two HIP events recorded on the stream it is
 * launched on, so the measured span is that kernel's time on its stream.
 * Disabled by default; enabling costs two event records per launch.
 * Process-wide and thread-safe. */
void evoattn_timing_enable(int enable);

/* Waits for every recorded launch to finish, then writes up to max_entries
 * aggregated records -- kernel name (NUL-terminated, at most 63 chars, in
 * names[i*64]), launch count and total milliseconds -- clears the record and
 * returns the number of distinct kernels seen (which may exceed max_entries),
 * or -1 if HIP reports an error while reading the events. */
int evoattn_timing_collect(int max_entries, char* names, int64_t* counts, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* EVOATTN_H */
