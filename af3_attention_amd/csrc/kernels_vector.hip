// Vector-ALU kernels for pair-biased 3D attention: one lane per softmax row
// (forward, dQ) or per key (dK/dV) or per bias element (dBias), fp32 math,
// fp32 or bf16 storage.  These serve the fp32 mode and every head_dim; the
// bf16 MFMA kernels are the fast path for bf16.
//
// The method is the memory-efficient attention of the MegaFold pages
// (gist.science technical summary, Methodik section 1 "EvoFlash-3D"): logits
// are formed tile by tile in on-chip memory and normalised with an online
// softmax (Milakov and Gimelshein, "Online normalizer calculation for
// softmax"), forward and backward, so the R*H*N*N logit tensor never exists in
// HBM.  The backward recomputes the softmax from the saved logsumexp.

#include "evoattn_internal.h"

namespace evo {
namespace {

constexpr int kTile = 64;  // keys (or queries) staged in LDS per step; one wave per block

__device__ __forceinline__ int64_t elem_offset(const Problem& p, int r, int pos, int h) {
  return ((static_cast<int64_t>(r) * p.row_stride + static_cast<int64_t>(pos) * p.pos_stride) * p.H + h) *
         p.D;
}

// Forward: block = one wave, 64 queries of one (row, head); grid flattened over
// (query block, head, row).
template <typename T, int D>
__global__ __launch_bounds__(kTile) void fwd_vector_kernel(Problem p, FwdArgs a) {
  __shared__ float ks[kTile][D + 1];
  __shared__ float vs[kTile][D + 1];
  __shared__ float ms[kTile];

  const int nqb = (p.N + kTile - 1) / kTile;
  int blk = blockIdx.x;
  const int qb = blk % nqb; blk /= nqb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int t = threadIdx.x;
  const int j = qb * kTile + t;
  const bool active = j < p.N;

  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* bias = static_cast<const T*>(a.bias);

  float qr[D], acc[D];
  const int64_t qoff = active ? elem_offset(p, r, j, h) : 0;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = active ? Elem<T>::load(q, qoff + c) * p.scale : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int kb = 0; kb < p.N; kb += kTile) {
    const int key = kb + t;
    if (key < p.N) {
      const int64_t off = elem_offset(p, r, key, h);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        ks[t][c] = Elem<T>::load(k, off + c);
        vs[t][c] = Elem<T>::load(v, off + c);
      }
      ms[t] = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
    }
    __syncthreads();
    const int kn = min(kTile, p.N - kb);
    if (active) {
      const int64_t brow = (static_cast<int64_t>(h) * p.N + j) * p.N + kb;
      for (int kk = 0; kk < kn; ++kk) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s += qr[c] * ks[kk][c];
        if (bias) s += Elem<T>::load(bias, brow + kk);
        s += ms[kk];
        if (s == -INFINITY) continue;
        if (s > m) {
          const float alpha = __expf(m - s);
          l = l * alpha + 1.f;
#pragma unroll
          for (int c = 0; c < D; ++c) acc[c] = acc[c] * alpha + vs[kk][c];
          m = s;
        } else {
          const float pr = __expf(s - m);
          l += pr;
#pragma unroll
          for (int c = 0; c < D; ++c) acc[c] += pr * vs[kk][c];
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  T* o = static_cast<T*>(a.o);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) Elem<T>::store(o, qoff + c, acc[c] * inv);
  if (a.lse) a.lse[(static_cast<int64_t>(r) * p.H + h) * p.N + j] = l > 0.f ? m + __logf(l) : -INFINITY;
}

// delta[r,h,j] = sum_c dout[r,j,h,c] * o[r,j,h,c]; one lane per softmax row.
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(Problem p, BwdArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(p.R) * p.H * p.N;
  if (idx >= total) return;
  const int j = static_cast<int>(idx % p.N);
  const int h = static_cast<int>((idx / p.N) % p.H);
  const int r = static_cast<int>(idx / (static_cast<int64_t>(p.N) * p.H));
  const int64_t off = elem_offset(p, r, j, h);
  const T* o = static_cast<const T*>(a.o);
  const T* dout = static_cast<const T*>(a.dout);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) s += Elem<T>::load(dout, off + c) * Elem<T>::load(o, off + c);
  a.delta[idx] = s;
}

// dQ: one lane per query; loops over key tiles staged in LDS.
template <typename T, int D>
__global__ __launch_bounds__(kTile) void dq_vector_kernel(Problem p, BwdArgs a) {
  __shared__ float ks[kTile][D + 1];
  __shared__ float vs[kTile][D + 1];
  __shared__ float ms[kTile];
  const int nqb = (p.N + kTile - 1) / kTile;
  int blk = blockIdx.x;
  const int qb = blk % nqb; blk /= nqb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int t = threadIdx.x;
  const int j = qb * kTile + t;
  const bool active = j < p.N;

  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* bias = static_cast<const T*>(a.bias);
  const T* dout = static_cast<const T*>(a.dout);

  const int64_t qoff = active ? elem_offset(p, r, j, h) : 0;
  float qr[D], dor[D], dq[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = active ? Elem<T>::load(q, qoff + c) * p.scale : 0.f;
    dor[c] = active ? Elem<T>::load(dout, qoff + c) : 0.f;
    dq[c] = 0.f;
  }
  const int64_t rowid = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
  const float lse = active ? a.lse[rowid] : -INFINITY;
  const float dlt = active ? a.delta[rowid] : 0.f;
  const bool live = active && lse != -INFINITY;

  for (int kb = 0; kb < p.N; kb += kTile) {
    const int key = kb + t;
    if (key < p.N) {
      const int64_t off = elem_offset(p, r, key, h);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        ks[t][c] = Elem<T>::load(k, off + c);
        vs[t][c] = Elem<T>::load(v, off + c);
      }
      ms[t] = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
    }
    __syncthreads();
    const int kn = min(kTile, p.N - kb);
    if (live) {
      const int64_t brow = (static_cast<int64_t>(h) * p.N + j) * p.N + kb;
      for (int kk = 0; kk < kn; ++kk) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s += qr[c] * ks[kk][c];
          dp += dor[c] * vs[kk][c];
        }
        if (bias) s += Elem<T>::load(bias, brow + kk);
        s += ms[kk];
        const float pr = s == -INFINITY ? 0.f : __expf(s - lse);
        const float ds = pr * (dp - dlt);
#pragma unroll
        for (int c = 0; c < D; ++c) dq[c] += ds * ks[kk][c];
      }
    }
    __syncthreads();
  }
  if (!active) return;
  T* dqo = static_cast<T*>(a.dq);
#pragma unroll
  for (int c = 0; c < D; ++c) Elem<T>::store(dqo, qoff + c, dq[c] * p.scale);
}

// dK, dV: one lane per key; loops over query tiles staged in LDS.
template <typename T, int D>
__global__ __launch_bounds__(kTile) void dkdv_vector_kernel(Problem p, BwdArgs a) {
  __shared__ float qs[kTile][D + 1];
  __shared__ float dos[kTile][D + 1];
  __shared__ float lses[kTile];
  __shared__ float dls[kTile];
  const int nkb = (p.N + kTile - 1) / kTile;
  int blk = blockIdx.x;
  const int kbk = blk % nkb; blk /= nkb;
  const int h = blk % p.H;
  const int r = blk / p.H;
  const int t = threadIdx.x;
  const int key = kbk * kTile + t;
  const bool active = key < p.N;

  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* bias = static_cast<const T*>(a.bias);
  const T* dout = static_cast<const T*>(a.dout);

  const int64_t koff = active ? elem_offset(p, r, key, h) : 0;
  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    kr[c] = active ? Elem<T>::load(k, koff + c) : 0.f;
    vr[c] = active ? Elem<T>::load(v, koff + c) : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const float mk = (active && a.mask) ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
  const bool live = active && mk != -INFINITY;

  for (int qb0 = 0; qb0 < p.N; qb0 += kTile) {
    const int j = qb0 + t;
    if (j < p.N) {
      const int64_t off = elem_offset(p, r, j, h);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        qs[t][c] = Elem<T>::load(q, off + c) * p.scale;
        dos[t][c] = Elem<T>::load(dout, off + c);
      }
      const int64_t rowid = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
      lses[t] = a.lse[rowid];
      dls[t] = a.delta[rowid];
    }
    __syncthreads();
    const int qn = min(kTile, p.N - qb0);
    if (live) {
      for (int jj = 0; jj < qn; ++jj) {
        const float lse = lses[jj];
        if (lse == -INFINITY) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
          s += qs[jj][c] * kr[c];
          dp += dos[jj][c] * vr[c];
        }
        if (bias) s += Elem<T>::load(bias, (static_cast<int64_t>(h) * p.N + qb0 + jj) * p.N + key);
        s += mk;
        const float pr = __expf(s - lse);
        const float ds = pr * (dp - dls[jj]);
#pragma unroll
        for (int c = 0; c < D; ++c) {
          dv[c] += pr * dos[jj][c];
          dk[c] += ds * qs[jj][c];
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  T* dko = static_cast<T*>(a.dk);
  T* dvo = static_cast<T*>(a.dv);
  // qs already carries the 1/sqrt(d) factor, so dk needs no further scaling.
#pragma unroll
  for (int c = 0; c < D; ++c) {
    Elem<T>::store(dko, koff + c, dk[c]);
    Elem<T>::store(dvo, koff + c, dv[c]);
  }
}

// dBias[h,j,k] = sum_r dS[r,h,j,k]: one lane per bias element, rows summed in
// increasing r, so the result is bit-identical on every call.
template <typename T, int D>
__global__ __launch_bounds__(kTile) void dbias_vector_kernel(Problem p, BwdArgs a) {
  const int nkb = (p.N + kTile - 1) / kTile;
  int blk = blockIdx.x;
  const int kbk = blk % nkb; blk /= nkb;
  const int j = blk % p.N;
  const int h = blk / p.N;
  const int key = kbk * kTile + threadIdx.x;
  if (key >= p.N) return;

  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* bias = static_cast<const T*>(a.bias);
  const T* dout = static_cast<const T*>(a.dout);
  const int64_t bidx = (static_cast<int64_t>(h) * p.N + j) * p.N + key;
  const float b = bias ? Elem<T>::load(bias, bidx) : 0.f;

  float acc = 0.f;
  for (int r = 0; r < p.R; ++r) {
    const int64_t rowid = (static_cast<int64_t>(r) * p.H + h) * p.N + j;
    const float lse = a.lse[rowid];
    const float mk = a.mask ? a.mask[static_cast<int64_t>(r) * p.N + key] : 0.f;
    if (lse == -INFINITY || mk == -INFINITY) continue;
    const int64_t qoff = elem_offset(p, r, j, h);
    const int64_t koff = elem_offset(p, r, key, h);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      s += Elem<T>::load(q, qoff + c) * Elem<T>::load(k, koff + c);
      dp += Elem<T>::load(dout, qoff + c) * Elem<T>::load(v, koff + c);
    }
    s = s * p.scale + b + mk;
    const float pr = __expf(s - lse);
    acc += pr * (dp - a.delta[rowid]);
  }
  a.dbias[bidx] = acc;
}

template <typename T, int D>
hipError_t fwd_vector_dispatch(const Problem& p, const FwdArgs& a, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>((p.N + kTile - 1) / kTile) * p.H * p.R;
  KernelTimer timer("fwd_vector", s);
  hipLaunchKernelGGL((fwd_vector_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(kTile), 0, s, p, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_vector_dispatch(const Problem& p, const BwdArgs& a, hipStream_t s) {
  const int64_t rows_total = static_cast<int64_t>(p.R) * p.H * p.N;
  hipError_t e;
  {
    KernelTimer timer("bwd_delta", s);
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3(static_cast<unsigned>((rows_total + 255) / 256)), dim3(256), 0,
                       s, p, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t blocks = static_cast<int64_t>((p.N + kTile - 1) / kTile) * p.H * p.R;
  {
    KernelTimer timer("bwd_dq_vector", s);
    hipLaunchKernelGGL((dq_vector_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(kTile), 0, s, p, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    KernelTimer timer("bwd_dkdv_vector", s);
    hipLaunchKernelGGL((dkdv_vector_kernel<T, D>), dim3(static_cast<unsigned>(blocks)), dim3(kTile), 0, s, p, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.dbias) {
    const int64_t bblocks = static_cast<int64_t>((p.N + kTile - 1) / kTile) * p.N * p.H;
    KernelTimer timer("bwd_dbias_vector", s);
    hipLaunchKernelGGL((dbias_vector_kernel<T, D>), dim3(static_cast<unsigned>(bblocks)), dim3(kTile), 0, s, p, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
hipError_t fwd_by_dim(const Problem& p, const FwdArgs& a, hipStream_t s) {
  switch (p.D) {
    case 8: return fwd_vector_dispatch<T, 8>(p, a, s);
    case 16: return fwd_vector_dispatch<T, 16>(p, a, s);
    case 32: return fwd_vector_dispatch<T, 32>(p, a, s);
    case 64: return fwd_vector_dispatch<T, 64>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t bwd_by_dim(const Problem& p, const BwdArgs& a, hipStream_t s) {
  switch (p.D) {
    case 8: return bwd_vector_dispatch<T, 8>(p, a, s);
    case 16: return bwd_vector_dispatch<T, 16>(p, a, s);
    case 32: return bwd_vector_dispatch<T, 32>(p, a, s);
    case 64: return bwd_vector_dispatch<T, 64>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_vector(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.dtype == 0 ? fwd_by_dim<float>(p, a, s) : fwd_by_dim<uint16_t>(p, a, s);
}

hipError_t launch_bwd_vector(const Problem& p, const BwdArgs& a, hipStream_t s) {
  return p.dtype == 0 ? bwd_by_dim<float>(p, a, s) : bwd_by_dim<uint16_t>(p, a, s);
}

}  // namespace evo
