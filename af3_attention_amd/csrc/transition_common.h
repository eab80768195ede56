// Building blocks shared by the SwiGLU transition kernels: the weight-chunk
// layout in LDS, its staging by direct global -> LDS copies, and silu.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_common.h"
#include "pipe_common.h"

namespace evo {
namespace trans {

using namespace mfma;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHC = 64;  // hidden units per weight chunk

template <int KS>
struct TransLayout {
  static constexpr int C = 16 * KS;
  static constexpr int PW = 2 * C + 16;    // bytes per w_a / w_b chunk row (one hidden unit)
  static constexpr int PO = 2 * kHC + 16;  // bytes per w_out chunk row (one channel)
  static constexpr int WA = 0, WB = kHC * PW, WO = 2 * kHC * PW;
  static constexpr int CHUNK = 2 * kHC * PW + C * PO;
  static constexpr int PIECES = 2 * kHC * (C / 8) + C * (kHC / 8);  // 16-byte pieces per chunk
  static constexpr int NP = (PIECES + kThreads - 1) / kThreads;
  static constexpr size_t lds_bytes() { return 8 * C + 2 * static_cast<size_t>(CHUNK); }
};

__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.f + fast_exp2(-a * kLog2e));
}

// Direct global -> LDS copies of a weight chunk into the padded LDS image above.
// The image is copied in 1 KB slices, slice s by wave s % kWaves, lane l filling
// bytes 16 l .. 16 l + 15 of the slice.  The three parts of the image (w_a rows,
// w_b rows, w_out columns) start on 1 KB boundaries, so every slice reads one
// matrix: a uniform base (the part's chunk) plus a per-lane byte offset that is
// the same for every chunk.  A lane whose 16 bytes fall in a row's padding copies
// the row's first 16 bytes (padding is never read).  The copies count in vmcnt:
// a wave waits for its own copies, then a barrier publishes them.  NW waves share
// the slices.
template <int KS, int NW = kWaves>
struct WeightCopy {
  using L = TransLayout<KS>;
  static constexpr int C = L::C;
  static constexpr int SLICES = L::CHUNK / 1024;
  static constexpr int NIT = (SLICES + NW - 1) / NW;
  static_assert(L::CHUNK % 1024 == 0 && L::WB % 1024 == 0 && L::WO % 1024 == 0,
                "every part of the chunk image must be whole 1 KB slices");
  const char* wa;
  const char* wb;
  const char* wo;
  uint32_t voff[NIT];

  __device__ __forceinline__ static int part_of(int slice) {
    return slice * 1024 < L::WB ? 0 : (slice * 1024 < L::WO ? 1 : 2);
  }
  // wave is uniform; hidden = rows of w_a (columns of w_out).
  __device__ __forceinline__ void init(const void* w_a, const void* w_b, const void* w_out, int hidden, int wave,
                                       int lane) {
    wa = static_cast<const char*>(w_a);
    wb = static_cast<const char*>(w_b);
    wo = static_cast<const char*>(w_out);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int slice = it * NW + wave;
      int o = slice * 1024 + 16 * lane;
      uint32_t v = 0;
      if (slice < SLICES) {
        if (o < L::WO) {
          if (o >= L::WB) o -= L::WB;
          const int row = o / L::PW, g = (o - row * L::PW) / 16;
          v = static_cast<uint32_t>(row * (2 * C) + 16 * (g < C / 8 ? g : 0));
        } else {
          o -= L::WO;
          const int row = o / L::PO, g = (o - row * L::PO) / 16;
          v = static_cast<uint32_t>(row) * (2u * static_cast<uint32_t>(hidden)) + 16u * (g < kHC / 8 ? g : 0);
        }
      }
      voff[it] = v;
    }
  }
  // Issues this wave's copies of chunk ch into the image at LDS byte address dst.
  __device__ __forceinline__ void issue(int ch, uint32_t dst, int wave) const {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int slice = it * NW + wave;
      if (slice >= SLICES) break;
      const int part = part_of(slice);
      const char* base = part == 0   ? wa + static_cast<int64_t>(ch) * (kHC * 2 * C)
                         : part == 1 ? wb + static_cast<int64_t>(ch) * (kHC * 2 * C)
                                     : wo + static_cast<int64_t>(ch) * (2 * kHC);
      pipe::copy16_to_lds(pipe::uniform_ptr(base), voff[it], dst + static_cast<uint32_t>(slice) * 1024u);
    }
  }
};

}  // namespace trans
}  // namespace evo
