// Bias pre-pass of the bf16 MFMA kernels: the bias scaled by sqrt(d) in fp32, as
// 32 x 32 tiles in MFMA accumulator order (layout: pipe_common.h).

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

// Tiled layout (see pipe_common.h): one thread per output float.
template <typename T>
__global__ __launch_bounds__(256) void bias_tiles_kernel(Problem p, const T* __restrict__ bias, float* __restrict__ out,
                                                         int nt, int orientation) {
  const int64_t total = static_cast<int64_t>(p.H) * nt * nt * 1024;
  const float sd = sqrtf(static_cast<float>(p.D));
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int e = static_cast<int>(idx & 3);
    const int lane = static_cast<int>((idx >> 2) & 63);
    const int g = static_cast<int>((idx >> 8) & 3);
    const int64_t t = idx >> 10;
    const int kt = static_cast<int>(t % nt);
    const int qt = static_cast<int>((t / nt) % nt);
    const int h = static_cast<int>(t / (static_cast<int64_t>(nt) * nt));
    const int row = 8 * g + 4 * (lane >> 5) + e;  // accumulator row of register 4g+e
    const int col = lane & 31;
    const int j = qt * 32 + (orientation == 0 ? col : row);
    const int k = kt * 32 + (orientation == 0 ? row : col);
    float val;
    if (k >= p.N) {
      val = -INFINITY;
    } else if (j >= p.N || bias == nullptr) {
      val = 0.f;
    } else {
      val = sd * Elem<T>::load(bias, (static_cast<int64_t>(h) * p.N + j) * p.N + k);
    }
    out[idx] = val;
  }
}

}  // namespace

size_t tiled_bias_bytes(const Problem& p) {
  const int64_t nt = bias_tiles(p.N);
  return static_cast<size_t>(p.H) * nt * nt * 1024 * sizeof(float);
}

hipError_t launch_bias_tiles(const Problem& p, const void* bias, float* out, int orientation, hipStream_t s) {
  const int nt = bias_tiles(p.N);
  const int64_t total = static_cast<int64_t>(p.H) * nt * nt * 1024;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 8192));
  KernelTimer timer(orientation ? "bias_tiles_k" : "bias_tiles_q", s);
  hipLaunchKernelGGL((bias_tiles_kernel<uint16_t>), dim3(blocks), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), out, nt, orientation);
  return hipGetLastError();
}

}  // namespace evo
