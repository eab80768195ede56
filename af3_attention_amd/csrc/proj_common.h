// Device helpers shared by the layer norm + projection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "evoattn_internal.h"

namespace evo {
namespace proj {

// Token of slot i (0..31) of 32-token tile `tile`, or -1 past the end.  Row
// tiles take 32 consecutive tokens; column tiles take 32 consecutive a at one b,
// so a transposed bias is written in 64-byte runs.
__device__ __forceinline__ int64_t tile_token(const ProjProblem& p, int tile, int i) {
  if (!p.col_tiles) {
    const int64_t t = static_cast<int64_t>(tile) * 32 + i;
    return t < p.T ? t : -1;
  }
  const int nab = (p.A + 31) >> 5;
  const int b = tile / nab;
  const int a = (tile - b * nab) * 32 + i;
  return a < p.A ? static_cast<int64_t>(a) * p.B + b : -1;
}

// Position of token tok = a*B + b in one head's plane of the bias [H][A][B]:
// tok itself, or b*A + a when the bias is transposed (tokens < 2^31).
__device__ __forceinline__ int64_t bias_pos(const ProjProblem& p, int64_t tok) {
  if (!p.bias_transpose) return tok;
  const int t = static_cast<int>(tok);
  const int a = t / p.B;
  return static_cast<int64_t>(t - a * p.B) * p.A + a;
}

__device__ __forceinline__ int64_t bias_offset(const ProjProblem& p, int hb, int64_t tok) {
  return static_cast<int64_t>(hb) * p.T + bias_pos(p, tok);
}

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

}  // namespace proj
}  // namespace evo
