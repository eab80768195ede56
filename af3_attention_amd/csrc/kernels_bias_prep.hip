// Bias pre-passes of the bf16 MFMA kernels: the bias scaled by sqrt(d) in fp32,
// either as a padded row-major square or as 32 x 32 tiles in MFMA accumulator order.

#include <algorithm>

#include "pipe_common.h"

namespace evo {
namespace {

// out[h][j][k] = sqrt(d) * bias[h][j][k] for j, k < N; -inf for k >= N (padding keys
// never win the softmax); 0 for padding queries.  Row stride nk, nq rows per head.
// transpose_out writes out[h][k][j] instead (the layout the backward's S tiles need).
template <typename T>
__global__ __launch_bounds__(256) void bias_prep_kernel(Problem p, const T* __restrict__ bias, float* __restrict__ out,
                                                        int nq, int nk, int transpose_out) {
  const int64_t total = static_cast<int64_t>(p.H) * nq * nk;
  const float sd = sqrtf(static_cast<float>(p.D));
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int inner = static_cast<int>(idx % nk);
    const int outer = static_cast<int>((idx / nk) % nq);
    const int h = static_cast<int>(idx / (static_cast<int64_t>(nk) * nq));
    const int j = transpose_out ? inner : outer;
    const int k = transpose_out ? outer : inner;
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

int bias_pad(int n) { return (n + 127) / 128 * 128; }

hipError_t launch_bias_prep(const Problem& p, const void* bias, float* out, int np, int transpose_out,
                            hipStream_t s) {
  const int64_t total = static_cast<int64_t>(p.H) * np * np;
  const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 8192));
  KernelTimer timer(transpose_out ? "bias_prep_t" : "bias_prep", s);
  hipLaunchKernelGGL((bias_prep_kernel<uint16_t>), dim3(blocks), dim3(256), 0, s, p,
                     static_cast<const uint16_t*>(bias), out, np, np, transpose_out);
  return hipGetLastError();
}

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
