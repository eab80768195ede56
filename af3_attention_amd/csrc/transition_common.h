// Building blocks shared by the SwiGLU transition kernels: the weight-chunk
// layout in LDS and its staging through registers, and silu.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_common.h"

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

// One thread's share of a weight chunk (64 hidden units: rows of w_a and w_b, the
// matching columns of w_out), loaded to registers and then stored to LDS.
template <int KS>
struct WeightChunks {
  using L = TransLayout<KS>;
  static constexpr int C = L::C;
  const uint16_t* wa;
  const uint16_t* wb;
  const uint16_t* wo;
  int hidden;
  int tid;
  u32x4 r[L::NP];

  // Pieces [I0, I1) of this thread (all of them by default).
  template <int I0 = 0, int I1 = L::NP>
  __device__ __forceinline__ void load(int ch) {
    const int h0 = ch * kHC;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int idx = tid + i * kThreads;
      u32x4 v = {0, 0, 0, 0};
      if (idx < 2 * kHC * (C / 8)) {
        const int which = idx / (kHC * (C / 8));
        const int rr = idx - which * (kHC * (C / 8));
        const int hid = rr / (C / 8), piece = rr - hid * (C / 8);
        const uint16_t* src = which ? wb : wa;
        v = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(h0 + hid) * C + 8 * piece);
      } else if (idx < L::PIECES) {
        const int rr = idx - 2 * kHC * (C / 8);
        const int c = rr / (kHC / 8), piece = rr - c * (kHC / 8);
        v = *reinterpret_cast<const u32x4*>(wo + static_cast<int64_t>(c) * hidden + h0 + 8 * piece);
      }
      r[i] = v;
    }
  }
  template <int I0 = 0, int I1 = L::NP>
  __device__ __forceinline__ void store(char* dst) const {
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < 2 * kHC * (C / 8)) {
        const int which = idx / (kHC * (C / 8));
        const int rr = idx - which * (kHC * (C / 8));
        const int hid = rr / (C / 8), piece = rr - hid * (C / 8);
        *reinterpret_cast<u32x4*>(dst + (which ? L::WB : L::WA) + hid * L::PW + 16 * piece) = r[i];
      } else if (idx < L::PIECES) {
        const int rr = idx - 2 * kHC * (C / 8);
        const int c = rr / (kHC / 8), piece = rr - c * (kHC / 8);
        *reinterpret_cast<u32x4*>(dst + L::WO + c * L::PO + 16 * piece) = r[i];
      }
    }
  }
};

}  // namespace trans
}  // namespace evo
