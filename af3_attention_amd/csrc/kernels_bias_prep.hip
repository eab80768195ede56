// Bias pre-pass of the bf16 MFMA kernels: the bias scaled by sqrt(d) in fp32, as
// 32 x 32 tiles in MFMA accumulator order (layout: pipe_common.h).

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

// Tiled layout (see pipe_common.h).  One workgroup per 32 x 32 block (query tile
// qt, key tile kt) of one head: the block is read once (coalesced rows of 32 keys)
// into LDS, then written in the query-lane order to out_q and, if out_k is not
// NULL, in the key-lane order to out_k, each as 256 coalesced 16-byte stores.
template <typename T>
__global__ __launch_bounds__(256) void bias_tiles_kernel(Problem p, const T* __restrict__ bias, float* __restrict__ out_q,
                                                         float* __restrict__ out_k, int nt) {
  __shared__ float tile[32][33];  // [query][key], padded
  const int kt = blockIdx.x % nt;
  const int qt = (blockIdx.x / nt) % nt;
  const int h = blockIdx.x / (nt * nt);
  const float sd = sqrtf(static_cast<float>(p.D));
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int jj = (t >> 5) + 8 * i, kk = t & 31;
    const int j = qt * 32 + jj, k = kt * 32 + kk;
    float val;
    if (k >= p.N) {
      val = -INFINITY;
    } else if (j >= p.N || bias == nullptr) {
      val = 0.f;
    } else {
      val = sd * Elem<T>::load(bias, (static_cast<int64_t>(h) * p.N + j) * p.N + k);
    }
    tile[jj][kk] = val;
  }
  __syncthreads();
  // Thread t writes floats 4t..4t+3 of the tile: register group g = t / 64 of lane
  // l = t % 64, accumulator rows 8g + 4(l / 32) + e, column l % 32.
  const int g = t >> 6, lane = t & 63;
  const int row0 = 8 * g + 4 * (lane >> 5), col = lane & 31;
  const int64_t off = (((static_cast<int64_t>(h) * nt + qt) * nt + kt) * 1024) + 4 * t;
  // Query lanes: rows are keys, the column is the query.
  *reinterpret_cast<float4*>(out_q + off) =
      make_float4(tile[col][row0], tile[col][row0 + 1], tile[col][row0 + 2], tile[col][row0 + 3]);
  if (out_k)  // key lanes: rows are queries, the column is the key
    *reinterpret_cast<float4*>(out_k + off) =
        make_float4(tile[row0][col], tile[row0 + 1][col], tile[row0 + 2][col], tile[row0 + 3][col]);
}

}  // namespace

size_t tiled_bias_bytes(const Problem& p) {
  const int64_t nt = bias_tiles(p.N);
  return static_cast<size_t>(p.H) * nt * nt * 1024 * sizeof(float);
}

hipError_t launch_bias_tiles(const Problem& p, const void* bias, float* out_q, float* out_k, hipStream_t s) {
  const int nt = bias_tiles(p.N);
  const int64_t blocks = static_cast<int64_t>(p.H) * nt * nt;
  KernelTimer timer(out_k ? "bias_tiles_qk" : "bias_tiles_q", s);
  hipLaunchKernelGGL((bias_tiles_kernel<uint16_t>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), out_q, out_k, nt);
  return hipGetLastError();
}

}  // namespace evo
