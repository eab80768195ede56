// C entry points of the EvoAttention library: argument validation, workspace
// layout and kernel dispatch.  Declared in include/evoattn.h.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "evoattn.h"
#include "evofusion.h"
#include "evoattn_internal.h"

namespace {

thread_local std::string g_last_error;

evoattn_status_t fail(evoattn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates sizes and enums; fills `p`.
evoattn_status_t check_problem(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype,
                               int transpose, evo::Problem* p) {
  if (rows < 1 || n < 1 || heads < 1 || head_dim < 1)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (rows=%lld n=%lld heads=%lld head_dim=%lld)",
                (long long)rows, (long long)n, (long long)heads, (long long)head_dim);
  if (dtype != EVOATTN_FP32 && dtype != EVOATTN_BF16)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "dtype %d is not EVOATTN_FP32 or EVOATTN_BF16", dtype);
  if (transpose != 0 && transpose != 1)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "transpose must be 0 or 1, got %d", transpose);
  if (head_dim != 8 && head_dim != 16 && head_dim != 32 && head_dim != 64)
    return fail(EVOATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (8, 16, 32, 64)", (long long)head_dim);
  const double elems = static_cast<double>(rows) * n * heads * head_dim;
  const double bias_elems = static_cast<double>(heads) * n * n;
  if (elems >= 2147483648.0 || bias_elems >= 2147483648.0)
    return fail(EVOATTN_ERR_UNSUPPORTED, "problem too large: R*N*H*d=%.0f, H*N*N=%.0f (limit 2^31 each)", elems,
                bias_elems);
  if (p) {
    p->R = static_cast<int>(rows);
    p->N = static_cast<int>(n);
    p->H = static_cast<int>(heads);
    p->D = static_cast<int>(head_dim);
    p->dtype = dtype;
    p->transpose = transpose;
    p->row_stride = transpose ? 1 : n;
    p->pos_stride = transpose ? rows : 1;
    p->scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  }
  return EVOATTN_OK;
}

#define REQUIRE_PTR(ptr, align)                                                                          \
  do {                                                                                                   \
    if (!(ptr)) return fail(EVOATTN_ERR_INVALID_ARGUMENT, "%s must not be NULL", #ptr);                   \
    if (!aligned((ptr), (align)))                                                                        \
      return fail(EVOATTN_ERR_INVALID_ARGUMENT, "%s must be %d-byte aligned", #ptr, (int)(align));        \
  } while (0)

#define OPTIONAL_PTR(ptr, align)                                                                         \
  do {                                                                                                   \
    if ((ptr) && !aligned((ptr), (align)))                                                               \
      return fail(EVOATTN_ERR_INVALID_ARGUMENT, "%s must be %d-byte aligned", #ptr, (int)(align));        \
  } while (0)

evoattn_status_t check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  return EVOATTN_OK;
}

// fp32 storage runs the vector-ALU kernels; bf16 storage runs the MFMA kernels.
bool use_mfma(const evo::Problem& p) { return p.dtype == EVOATTN_BF16; }

size_t fwd_ws_bytes(const evo::Problem& p) { return use_mfma(p) ? round_up(evo::fwd_mfma_workspace_bytes(p)) : 0; }

size_t bwd_ws_bytes(const evo::Problem& p) {
  if (use_mfma(p)) return round_up(evo::bwd_mfma_workspace_bytes(p));
  const size_t delta = static_cast<size_t>(p.R) * p.H * p.N * sizeof(float);
  return round_up(delta);
}

// Validates the layer norm + projection problem; fills `p`.
evoattn_status_t check_proj(int64_t A, int64_t B, int64_t C, int64_t heads, int64_t head_dim, int dtype,
                            int bias_transpose, float eps, bool with_qkv, bool with_bias, evo::ProjProblem* p) {
  if (A < 1 || B < 1 || C < 1 || heads < 1 || head_dim < 1)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (a=%lld b=%lld channels=%lld heads=%lld head_dim=%lld)",
                (long long)A, (long long)B, (long long)C, (long long)heads, (long long)head_dim);
  if (dtype != EVOATTN_FP32 && dtype != EVOATTN_BF16)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "dtype %d is not EVOATTN_FP32 or EVOATTN_BF16", dtype);
  if (bias_transpose != 0 && bias_transpose != 1)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "bias_transpose must be 0 or 1, got %d", bias_transpose);
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0, got %g", (double)eps);
  if (!with_qkv && !with_bias)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "w_qkv and w_bias are both NULL: nothing to project");
  if (head_dim != 8 && head_dim != 16 && head_dim != 32 && head_dim != 64)
    return fail(EVOATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (8, 16, 32, 64)", (long long)head_dim);
  if (C < 16 || C > 2048 || C % 8 != 0)
    return fail(EVOATTN_ERR_UNSUPPORTED, "channels %lld not supported (a multiple of 8 in 16..2048)", (long long)C);
  if (with_bias && A != B)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "the pair bias needs a square token grid, got a=%lld b=%lld",
                (long long)A, (long long)B);
  const double T = static_cast<double>(A) * B;
  const double widest = std::max(static_cast<double>(C), 3.0 * heads * head_dim);
  if (T >= 2147483648.0 || T * widest >= 2147483648.0 || heads * head_dim * 3 >= 65536)
    return fail(EVOATTN_ERR_UNSUPPORTED, "problem too large: tokens=%.0f, widest row=%.0f", T, widest);
  if (p) {
    p->A = static_cast<int>(A);
    p->B = static_cast<int>(B);
    p->C = static_cast<int>(C);
    p->H = static_cast<int>(heads);
    p->D = static_cast<int>(head_dim);
    p->T = A * B;
    p->dtype = dtype;
    p->bias_transpose = bias_transpose;
    p->n_qkv = with_qkv ? static_cast<int>(3 * heads * head_dim) : 0;
    p->n_out = p->n_qkv + (with_bias ? static_cast<int>(heads) : 0);
    p->col_tiles = (with_bias && bias_transpose) ? 1 : 0;
    p->tiles = p->col_tiles ? static_cast<int>(((A + 31) / 32) * B) : static_cast<int>((A * B + 31) / 32);
    p->eps = eps;
  }
  return EVOATTN_OK;
}

// Validates the SwiGLU transition problem; fills `p`.
evoattn_status_t check_transition(int64_t A, int64_t B, int64_t C, int64_t expansion, int dtype, float eps,
                                  evo::TransProblem* p) {
  if (A < 1 || B < 1 || C < 1 || expansion < 1)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (a=%lld b=%lld channels=%lld expansion=%lld)",
                (long long)A, (long long)B, (long long)C, (long long)expansion);
  if (dtype != EVOATTN_FP32 && dtype != EVOATTN_BF16)
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "dtype %d is not EVOATTN_FP32 or EVOATTN_BF16", dtype);
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0, got %g", (double)eps);
  if (dtype != EVOATTN_BF16)
    return fail(EVOATTN_ERR_UNSUPPORTED, "the transition is implemented for bf16 only");
  if (C != 64 && C != 128)
    return fail(EVOATTN_ERR_UNSUPPORTED, "channels %lld not supported (64 or 128)", (long long)C);
  if (expansion > 16)
    return fail(EVOATTN_ERR_UNSUPPORTED, "expansion %lld not supported (1..16)", (long long)expansion);
  const double T = static_cast<double>(A) * B;
  if (T * C >= 2147483648.0 || T * C * expansion >= 4294967296.0)
    return fail(EVOATTN_ERR_UNSUPPORTED, "problem too large: tokens=%.0f", T);
  if (p) {
    p->A = static_cast<int>(A);
    p->B = static_cast<int>(B);
    p->C = static_cast<int>(C);
    p->hidden = static_cast<int>(expansion * C);
    p->T = A * B;
    p->tiles = static_cast<int>((A * B + 31) / 32);
    p->eps = eps;
  }
  return EVOATTN_OK;
}

// Scratch of evoattn_fwd_noalloc: a file-scope device array, so that the entry
// point needs no allocation.  Every device that runs the library holds its own
// copy until the process ends.  In host code `scratch` only names the symbol;
// its device address (one per device) comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = EVOATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
evoattn_status_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(EVOATTN_ERR_DEVICE, "device index %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(EVOATTN_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EVOATTN_OK;
}

}  // namespace

extern "C" {

int evoattn_abi_version(void) { return EVOATTN_ABI_VERSION; }

const char* evoattn_status_string(int status) {
  switch (status) {
    case EVOATTN_OK: return "EVOATTN_OK";
    case EVOATTN_ERR_INVALID_ARGUMENT: return "EVOATTN_ERR_INVALID_ARGUMENT";
    case EVOATTN_ERR_UNSUPPORTED: return "EVOATTN_ERR_UNSUPPORTED";
    case EVOATTN_ERR_WORKSPACE: return "EVOATTN_ERR_WORKSPACE";
    case EVOATTN_ERR_DEVICE: return "EVOATTN_ERR_DEVICE";
    default: return "EVOATTN_UNKNOWN_STATUS";
  }
}

const char* evoattn_last_error_detail(void) { return g_last_error.c_str(); }

size_t evoattn_fwd_workspace_bytes(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype) {
  evo::Problem p;
  if (check_problem(rows, n, heads, head_dim, dtype, 0, &p) != EVOATTN_OK) return 0;
  return fwd_ws_bytes(p);
}

size_t evoattn_bwd_workspace_bytes(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype) {
  evo::Problem p;
  if (check_problem(rows, n, heads, head_dim, dtype, 0, &p) != EVOATTN_OK) return 0;
  return bwd_ws_bytes(p);
}

evoattn_status_t evoattn_fwd(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype, int transpose,
                             const void* q, const void* k, const void* v, const void* bias, const float* mask,
                             void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  evo::Problem p;
  evoattn_status_t st = check_problem(rows, n, heads, head_dim, dtype, transpose, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(k, 16);
  REQUIRE_PTR(v, 16);
  REQUIRE_PTR(o, 16);
  OPTIONAL_PTR(bias, 16);
  OPTIONAL_PTR(mask, 4);
  OPTIONAL_PTR(lse, 4);
  const size_t need = fwd_ws_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EVOATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu at %p", need, workspace_bytes, workspace);
  if (workspace && !aligned(workspace, 256))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((st = check_device()) != EVOATTN_OK) return st;

  evo::FwdArgs a{q, k, v, bias, mask, o, lse};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = use_mfma(p) ? evo::launch_fwd_mfma(p, a, workspace, s) : evo::launch_fwd_vector(p, a, s);
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "forward launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

evoattn_status_t evoattn_fwd_noalloc(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype,
                                     int transpose, const void* q, const void* k, const void* v, const void* bias,
                                     const float* mask, void* o, float* lse, void* stream) {
  evo::Problem p;
  evoattn_status_t st = check_problem(rows, n, heads, head_dim, dtype, transpose, &p);
  if (st != EVOATTN_OK) return st;
  const size_t need = fwd_ws_bytes(p);
  if (need > kNoAllocScratchBytes)
    return fail(EVOATTN_ERR_WORKSPACE,
                "problem needs %zu bytes of scratch; evoattn_fwd_noalloc holds at most %zu "
                "(EVOATTN_NOALLOC_SCRATCH_BYTES): call evoattn_fwd with a workspace instead",
                need, kNoAllocScratchBytes);
  if ((st = check_device()) != EVOATTN_OK) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != EVOATTN_OK) return st;
  return evoattn_fwd(rows, n, heads, head_dim, dtype, transpose, q, k, v, bias, mask, o, lse, ws,
                     kNoAllocScratchBytes, stream);
}

evoattn_status_t evoattn_bwd(int64_t rows, int64_t n, int64_t heads, int64_t head_dim, int dtype, int transpose,
                             const void* q, const void* k, const void* v, const void* bias, const float* mask,
                             const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             float* dbias, void* workspace, size_t workspace_bytes, void* stream) {
  evo::Problem p;
  evoattn_status_t st = check_problem(rows, n, heads, head_dim, dtype, transpose, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(k, 16);
  REQUIRE_PTR(v, 16);
  REQUIRE_PTR(o, 16);
  REQUIRE_PTR(lse, 4);
  REQUIRE_PTR(dout, 16);
  REQUIRE_PTR(dq, 16);
  REQUIRE_PTR(dk, 16);
  REQUIRE_PTR(dv, 16);
  OPTIONAL_PTR(bias, 16);
  OPTIONAL_PTR(mask, 4);
  OPTIONAL_PTR(dbias, 4);
  const size_t need = bwd_ws_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EVOATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu at %p", need, workspace_bytes, workspace);
  if (workspace && !aligned(workspace, 256))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((st = check_device()) != EVOATTN_OK) return st;

  evo::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.bias = bias; a.mask = mask; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dbias = dbias;
  a.delta = static_cast<float*>(workspace);
  a.scratch = nullptr;
  a.scratch_bytes = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = use_mfma(p) ? evo::launch_bwd_mfma(p, a, workspace, s) : evo::launch_bwd_vector(p, a, s);
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

evoattn_status_t evoattn_ln_proj_fwd(int64_t a, int64_t b, int64_t channels, int64_t heads, int64_t head_dim,
                                     int dtype, int bias_transpose, float eps, const void* x, const float* gamma,
                                     const float* beta, const void* w_qkv, const void* w_bias, void* q, void* k,
                                     void* v, void* bias, float* mean, float* rstd, void* stream) {
  evo::ProjProblem p;
  evoattn_status_t st = check_proj(a, b, channels, heads, head_dim, dtype, bias_transpose, eps, w_qkv != nullptr,
                                   w_bias != nullptr, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(gamma, 4);
  REQUIRE_PTR(beta, 4);
  if (w_qkv) {
    REQUIRE_PTR(w_qkv, 16);
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(v, 16);
  } else if (q || k || v) {
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "q, k, v must be NULL when w_qkv is NULL");
  }
  if (w_bias) {
    REQUIRE_PTR(w_bias, 16);
    REQUIRE_PTR(bias, 16);
  } else if (bias) {
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "bias must be NULL when w_bias is NULL");
  }
  if ((mean == nullptr) != (rstd == nullptr))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "mean and rstd must both be given or both be NULL");
  OPTIONAL_PTR(mean, 4);
  OPTIONAL_PTR(rstd, 4);
  if ((st = check_device()) != EVOATTN_OK) return st;

  evo::ProjFwdArgs args{x, gamma, beta, w_qkv, w_bias, q, k, v, bias, mean, rstd};
  hipError_t e = evo::launch_ln_proj_fwd(p, args, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "layer norm + projection launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

size_t evoattn_ln_proj_bwd_workspace_bytes(int64_t a, int64_t b, int64_t channels, int64_t heads, int64_t head_dim,
                                           int dtype, int with_qkv, int with_bias) {
  evo::ProjProblem p;
  if (check_proj(a, b, channels, heads, head_dim, dtype, 0, 0.f, with_qkv != 0, with_bias != 0, &p) != EVOATTN_OK)
    return 0;
  return round_up(evo::ln_proj_bwd_workspace_bytes(p));
}

evoattn_status_t evoattn_ln_proj_bwd(int64_t a, int64_t b, int64_t channels, int64_t heads, int64_t head_dim,
                                     int dtype, int bias_transpose, const void* x, const float* gamma,
                                     const float* beta, const void* w_qkv, const void* w_bias, const float* mean,
                                     const float* rstd, const void* dq, const void* dk, const void* dv,
                                     const float* dbias, void* dx, float* dgamma, float* dbeta, float* dw_qkv,
                                     float* dw_bias, void* workspace, size_t workspace_bytes, void* stream) {
  evo::ProjProblem p;
  evoattn_status_t st = check_proj(a, b, channels, heads, head_dim, dtype, bias_transpose, 0.f, w_qkv != nullptr,
                                   w_bias != nullptr, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(gamma, 4);
  REQUIRE_PTR(beta, 4);
  REQUIRE_PTR(mean, 4);
  REQUIRE_PTR(rstd, 4);
  REQUIRE_PTR(dx, 16);
  REQUIRE_PTR(dgamma, 4);
  REQUIRE_PTR(dbeta, 4);
  if (w_qkv) {
    REQUIRE_PTR(w_qkv, 16);
    REQUIRE_PTR(dq, 16);
    REQUIRE_PTR(dk, 16);
    REQUIRE_PTR(dv, 16);
    REQUIRE_PTR(dw_qkv, 4);
  } else if (dq || dk || dv || dw_qkv) {
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "dq, dk, dv and dw_qkv must be NULL when w_qkv is NULL");
  }
  if (w_bias) {
    REQUIRE_PTR(w_bias, 16);
    REQUIRE_PTR(dbias, 4);
    REQUIRE_PTR(dw_bias, 4);
  } else if (dbias || dw_bias) {
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "dbias and dw_bias must be NULL when w_bias is NULL");
  }
  const size_t need = round_up(evo::ln_proj_bwd_workspace_bytes(p));
  if (!workspace || workspace_bytes < need)
    return fail(EVOATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu at %p", need, workspace_bytes, workspace);
  if (!aligned(workspace, 256)) return fail(EVOATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((st = check_device()) != EVOATTN_OK) return st;

  evo::ProjBwdArgs args{x, gamma, beta, w_qkv, w_bias, mean, rstd, dq, dk, dv, dbias, dx, dgamma, dbeta, dw_qkv, dw_bias};
  hipError_t e = evo::launch_ln_proj_bwd(p, args, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(EVOATTN_ERR_DEVICE, "layer norm + projection backward launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

evoattn_status_t evoattn_transition_fwd(int64_t a, int64_t b, int64_t channels, int64_t expansion, int dtype,
                                        float eps, const void* x, const float* gamma, const float* beta,
                                        const void* w_a, const void* w_b, const void* w_out, void* out, float* mean,
                                        float* rstd, void* stream) {
  evo::TransProblem p;
  evoattn_status_t st = check_transition(a, b, channels, expansion, dtype, eps, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(gamma, 4);
  REQUIRE_PTR(beta, 4);
  REQUIRE_PTR(w_a, 16);
  REQUIRE_PTR(w_b, 16);
  REQUIRE_PTR(w_out, 16);
  REQUIRE_PTR(out, 16);
  if ((mean == nullptr) != (rstd == nullptr))
    return fail(EVOATTN_ERR_INVALID_ARGUMENT, "mean and rstd must both be given or both be NULL");
  OPTIONAL_PTR(mean, 4);
  OPTIONAL_PTR(rstd, 4);
  if ((st = check_device()) != EVOATTN_OK) return st;
  evo::TransFwdArgs args{x, gamma, beta, w_a, w_b, w_out, out, mean, rstd};
  hipError_t e = evo::launch_transition_fwd(p, args, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "transition launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

size_t evoattn_transition_bwd_workspace_bytes(int64_t a, int64_t b, int64_t channels, int64_t expansion, int dtype) {
  evo::TransProblem p;
  if (check_transition(a, b, channels, expansion, dtype, 0.f, &p) != EVOATTN_OK) return 0;
  return round_up(evo::transition_bwd_workspace_bytes(p));
}

evoattn_status_t evoattn_transition_bwd(int64_t a, int64_t b, int64_t channels, int64_t expansion, int dtype,
                                        const void* x, const float* gamma, const float* beta, const void* w_a,
                                        const void* w_b, const void* w_out, const float* mean, const float* rstd,
                                        const void* dout, void* dx, float* dgamma, float* dbeta, float* dw_a,
                                        float* dw_b, float* dw_out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  evo::TransProblem p;
  evoattn_status_t st = check_transition(a, b, channels, expansion, dtype, 0.f, &p);
  if (st != EVOATTN_OK) return st;
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(gamma, 4);
  REQUIRE_PTR(beta, 4);
  REQUIRE_PTR(w_a, 16);
  REQUIRE_PTR(w_b, 16);
  REQUIRE_PTR(w_out, 16);
  REQUIRE_PTR(mean, 4);
  REQUIRE_PTR(rstd, 4);
  REQUIRE_PTR(dout, 16);
  REQUIRE_PTR(dx, 16);
  REQUIRE_PTR(dgamma, 4);
  REQUIRE_PTR(dbeta, 4);
  REQUIRE_PTR(dw_a, 4);
  REQUIRE_PTR(dw_b, 4);
  REQUIRE_PTR(dw_out, 4);
  const size_t need = round_up(evo::transition_bwd_workspace_bytes(p));
  if (!workspace || workspace_bytes < need)
    return fail(EVOATTN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu at %p", need, workspace_bytes, workspace);
  if (!aligned(workspace, 256)) return fail(EVOATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((st = check_device()) != EVOATTN_OK) return st;
  evo::TransBwdArgs args{x, gamma, beta, w_a, w_b, w_out, mean, rstd, dout, dx, dgamma, dbeta, dw_a, dw_b, dw_out};
  hipError_t e = evo::launch_transition_bwd(p, args, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(EVOATTN_ERR_DEVICE, "transition backward launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return EVOATTN_OK;
}

}  // extern "C"
