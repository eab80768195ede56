// Bias pre-pass of the bf16 MFMA kernels: the bias scaled by sqrt(d) in fp32, as
// 32 x 32 tiles in MFMA accumulator order (layout: pipe_common.h).

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

// Tiled layout (see pipe_common.h).  One workgroup per 32 x 32 block (query tile
// qt, key tile kt) of one head.
template <typename T>
__global__ __launch_bounds__(256) void bias_tiles_kernel(Problem p, const T* __restrict__ bias, float* __restrict__ out_q,
                                                         float* __restrict__ out_k, int nt) {
  pipe::bias_tile(p, bias, out_q, out_k, nt, blockIdx.x);
}

// Forward pre-pass: the bias tiles in the query-lane order (blocks 0 .. tiles - 1)
// and, with a mask, one block per attention row r: the key-side split operand of
// sqrt(d) * mask[r][k] for every key (pipe::key_aug's layout in all 16 bytes,
// with a masked key's -inf kept exact) and the last key of the row that is not
// masked (-1 if there is none).
template <typename T>
__global__ __launch_bounds__(256) void fwd_prep_kernel(Problem p, const T* __restrict__ bias, const float* __restrict__ mask,
                                                       float* __restrict__ out_q, uint4* __restrict__ kaug,
                                                       int* __restrict__ last_live, int nt, int tiles) {
  if (static_cast<int>(blockIdx.x) < tiles) {
    pipe::bias_tile(p, bias, out_q, static_cast<float*>(nullptr), nt, blockIdx.x);
    return;
  }
  __shared__ int red[4];
  const int r = blockIdx.x - tiles;
  const float sd = sqrtf(static_cast<float>(p.D));
  int last = -1;
  for (int k = threadIdx.x; k < p.N; k += 256) {
    const float m = mask[static_cast<int64_t>(r) * p.N + k];
    const float ms = sd * m;
    // A masked key carries -inf itself (one bf16 part; the others 0), so its
    // logit is exactly -inf.
    const pipe::Split3 sm = ms == -INFINITY ? pipe::Split3{0xff80u, 0u, 0u} : pipe::split3(ms);
    kaug[static_cast<int64_t>(r) * p.N + k] =
        make_uint4(pipe::kBf16One | (pipe::kBf16One << 16), pipe::kBf16One | (sm.hi << 16), sm.mid | (sm.lo << 16), 0u);
    if (m != -INFINITY) last = k;
  }
  for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = last;
  __syncthreads();
  if (threadIdx.x == 0) last_live[r] = max(max(red[0], red[1]), max(red[2], red[3]));
}

}  // namespace

size_t tiled_bias_bytes(const Problem& p) {
  const int64_t nt = bias_tiles(p.N);
  return static_cast<size_t>(p.H) * nt * nt * 1024 * sizeof(float);
}

hipError_t launch_bias_tiles(const Problem& p, const void* bias, float* out_q, float* out_k, hipStream_t s) {
  const int nt = bias_tiles(p.N);
  const int64_t blocks = static_cast<int64_t>(p.H) * nt * nt;
  KernelTimer timer(out_q ? (out_k ? "bias_tiles_qk" : "bias_tiles_q") : "bias_tiles_k", s);
  hipLaunchKernelGGL((bias_tiles_kernel<uint16_t>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), out_q, out_k, nt);
  return hipGetLastError();
}

hipError_t launch_fwd_prep(const Problem& p, const void* bias, const float* mask, float* out_q, void* kaug,
                           int* last_live, hipStream_t s) {
  const int nt = bias_tiles(p.N);
  const int tiles = p.H * nt * nt;
  const int64_t blocks = static_cast<int64_t>(tiles) + (mask ? p.R : 0);
  KernelTimer timer("fwd_prep", s);
  hipLaunchKernelGGL((fwd_prep_kernel<uint16_t>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), mask, out_q, static_cast<uint4*>(kaug), last_live, nt, tiles);
  return hipGetLastError();
}

}  // namespace evo
