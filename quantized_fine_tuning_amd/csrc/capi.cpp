// C ABI of the NF4 QLoRA library: argument validation (entirely on the host,
// before any HIP call), workspace sizing and dispatch to the kernel launchers.
// The declarations and their contracts are in include/qlora_nf4.h.
#include "qlora_nf4.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "host.h"

namespace {

thread_local std::string g_last_error;

qlora_status fail(qlora_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
qlora_status fail(qlora_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

qlora_status ok() {
  g_last_error.clear();
  return QLORA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define CHECK_PTR(p)                                                                        \
  do {                                                                                      \
    if ((p) == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);        \
    if (!aligned16(p)) return fail(QLORA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

#define CHECK_OPT_PTR(p)                                                                    \
  do {                                                                                      \
    if ((p) != nullptr && !aligned16(p))                                                    \
      return fail(QLORA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p);           \
  } while (0)

qlora_status check_shape(const char* fn, int64_t N, int64_t K) {
  if (N <= 0 || K <= 0)
    return fail(QLORA_ERR_INVALID_ARG, "%s: N=%lld and K=%lld must be positive", fn, (long long)N,
                (long long)K);
  if (K % 64 != 0)
    return fail(QLORA_ERR_INVALID_ARG, "%s: K=%lld is not a multiple of 64", fn, (long long)K);
  if (N % 8 != 0)
    return fail(QLORA_ERR_INVALID_ARG, "%s: N=%lld is not a multiple of 8", fn, (long long)N);
  if (N > (int64_t(1) << 40) / K)
    return fail(QLORA_ERR_INVALID_ARG, "%s: N*K too large", fn);
  return QLORA_OK;
}

qlora_status check_rank(const char* fn, int32_t r) {
  if (r < 1 || r > 256) return fail(QLORA_ERR_INVALID_ARG, "%s: r=%d outside [1, 256]", fn, r);
  return QLORA_OK;
}

qlora_status check_tensor(const char* fn, const qlora_nf4_t* q) {
  if (q == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: weight descriptor is NULL", fn);
  qlora_status st = check_shape(fn, q->n_rows, q->n_cols);
  if (st != QLORA_OK) return st;
  const uint8_t* codes = q->codes;
  const uint8_t* absmax_e4m3 = q->absmax_e4m3;
  const float* dq_scale = q->dq_scale;
  const float* dq_mean = q->dq_mean;
  CHECK_PTR(codes);
  CHECK_PTR(absmax_e4m3);
  CHECK_PTR(dq_scale);
  CHECK_PTR(dq_mean);
  return QLORA_OK;
}

// Limits of one linear pass, from the 32-bit byte offsets of the kernels'
// buffer loads (one buffer resource spans at most 2^31 - 1 bytes): the packed
// codes of the weight, the activations and gradients of one call, and the
// transposed hi/lo splits [2Rp, round_up(M, 64)] of the low-rank factors.
qlora_status check_linear_limits(const char* fn, int64_t M, int64_t N, int64_t K, int32_t r) {
  const int64_t lim = int64_t(1) << 31;
  if (N * K / 2 >= lim) return fail(QLORA_ERR_INVALID_ARG, "%s: N*K/2 = %lld code bytes (limit 2^31)", fn, (long long)(N * K / 2));
  const int64_t wide = N > K ? N : K;
  if (M > 0 && M >= (lim / 2) / wide)
    return fail(QLORA_ERR_INVALID_ARG, "%s: M*max(N, K) = %lld elements (limit 2^30)", fn, (long long)(M * wide));
  const int64_t Rp = (r + 31) / 32 * 32, Mp = (M + 63) / 64 * 64;
  if (2 * Rp * Mp * 2 >= lim)
    return fail(QLORA_ERR_INVALID_ARG, "%s: M=%lld too large for rank %d (2*Rp*Mp*2 >= 2^31)", fn, (long long)M, r);
  return QLORA_OK;
}

qlora_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(QLORA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

qnf4::Nf4View view(const qlora_nf4_t* q) {
  return qnf4::Nf4View{q->codes, q->absmax_e4m3, q->dq_scale, q->dq_mean, q->n_rows, q->n_cols};
}

}  // namespace

namespace qnf4 {
TimingHook& timing_hook() {
  thread_local TimingHook h{0, nullptr, nullptr};
  return h;
}
}  // namespace qnf4

extern "C" {

qlora_status qlora_nf4_sizes(int64_t N, int64_t K, int64_t M_max, int32_t r, qlora_sizes_t* out) {
  const char* fn = "qlora_nf4_sizes";
  if (out == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: out is NULL", fn);
  qlora_status st = check_shape(fn, N, K);
  if (st != QLORA_OK) return st;
  if ((st = check_rank(fn, r)) != QLORA_OK) return st;
  if (M_max < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: M_max=%lld < 0", fn, (long long)M_max);
  const int64_t nb = N * K / 64;
  out->codes_bytes = (size_t)(N * K / 2);
  out->absmax_bytes = (size_t)nb;
  out->scale_bytes = (size_t)(4 * ((nb + 255) / 256));
  out->mean_bytes = 4;
  out->quantize_ws_bytes = qnf4::quant_layout(N, K).total;
  out->fwd_ws_bytes = qnf4::fwd_ws_bytes_max(M_max, N, K, r);
  out->bwd_ws_bytes = qnf4::bwd_ws_bytes_max(M_max, N, K, r);
  return ok();
}

qlora_status qlora_nf4_quantize(const void* W, qlora_dtype w_dtype, int64_t N, int64_t K,
                                const qlora_nf4_t* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "qlora_nf4_quantize";
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: w_dtype=%d (expected F32 or BF16)", fn, w_dtype);
  qlora_status st = check_shape(fn, N, K);
  if (st != QLORA_OK) return st;
  CHECK_PTR(W);
  if ((st = check_tensor(fn, out)) != QLORA_OK) return st;
  if (out->n_rows != N || out->n_cols != K)
    return fail(QLORA_ERR_INVALID_ARG, "%s: descriptor shape %lldx%lld != %lldx%lld", fn,
                (long long)out->n_rows, (long long)out->n_cols, (long long)N, (long long)K);
  const qnf4::QuantLayout L = qnf4::quant_layout(N, K);
  if (ws_bytes < L.total)
    return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn, ws_bytes,
                L.total);
  CHECK_PTR(ws);
  return hip_status(fn, qnf4::launch_quantize(W, w_dtype == QLORA_BF16, N, K, out->codes,
                                              out->absmax_e4m3, out->dq_scale, out->dq_mean,
                                              static_cast<char*>(ws), L,
                                              static_cast<hipStream_t>(stream)));
}

qlora_status qlora_dequantize(const qlora_nf4_t* q, void* out, qlora_dtype out_dtype,
                              void* stream) {
  const char* fn = "qlora_dequantize";
  qlora_status st = check_tensor(fn, q);
  if (st != QLORA_OK) return st;
  if (out_dtype != QLORA_BF16 && out_dtype != QLORA_F16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: out_dtype=%d (BF16 or F16)", fn, out_dtype);
  CHECK_PTR(out);
  return hip_status(fn, qnf4::launch_dequantize(q->codes, q->absmax_e4m3, q->dq_scale, q->dq_mean,
                                                q->n_rows, q->n_cols, static_cast<uint16_t*>(out),
                                                out_dtype == QLORA_F16, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_linear_fwd(const qlora_nf4_t* W, const void* X, int64_t M, const void* A,
                              const void* B, int32_t r, float alpha, void* Y, qlora_dtype y_dtype,
                              float* T_save, void* ws, size_t ws_bytes, void* stream) {
  return qlora_linear_fwd_ex(W, X, M, A, B, r, alpha, Y, y_dtype, T_save, ws, ws_bytes, QLORA_BF16, stream);
}

}  // extern "C"

namespace {

// Arguments of a forward pass, everything but the workspace.
qlora_status check_fwd_args(const char* fn, const qlora_nf4_t* W, const void* X, int64_t M, const void* A,
                            const void* B, int32_t r, const void* Y, qlora_dtype y_dtype, const float* T_save,
                            qlora_dtype compute_dtype) {
  qlora_status st = check_tensor(fn, W);
  if (st != QLORA_OK) return st;
  if (compute_dtype != QLORA_BF16 && compute_dtype != QLORA_F16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: compute_dtype=%d (BF16 or F16)", fn, compute_dtype);
  if ((st = check_rank(fn, r)) != QLORA_OK) return st;
  if (M < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: M=%lld < 0", fn, (long long)M);
  if ((st = check_linear_limits(fn, M, W->n_rows, W->n_cols, r)) != QLORA_OK) return st;
  if (y_dtype != QLORA_F32 && y_dtype != compute_dtype)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: y_dtype=%d (F32 or the compute dtype)", fn, y_dtype);
  CHECK_PTR(A);
  CHECK_PTR(B);
  if (M > 0) {
    CHECK_PTR(X);
    CHECK_PTR(Y);
  }
  CHECK_OPT_PTR(T_save);
  return QLORA_OK;
}

// The static scratch of qlora_linear_fwd_noalloc: one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it passes the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

qlora_status qlora_linear_fwd_ex(const qlora_nf4_t* W, const void* X, int64_t M, const void* A,
                                 const void* B, int32_t r, float alpha, void* Y, qlora_dtype y_dtype,
                                 float* T_save, void* ws, size_t ws_bytes, qlora_dtype compute_dtype,
                                 void* stream) {
  const char* fn = "qlora_linear_fwd";
  qlora_status st = check_fwd_args(fn, W, X, M, A, B, r, Y, y_dtype, T_save, compute_dtype);
  if (st != QLORA_OK) return st;
  const qnf4::FwdLayout L = qnf4::fwd_layout(M, W->n_rows, W->n_cols, r);
  if (ws_bytes < L.total)
    return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn, ws_bytes,
                L.total);
  if (M > 0) CHECK_PTR(ws);
  return hip_status(fn, qnf4::launch_forward(
                            view(W), static_cast<const uint16_t*>(X), M,
                            static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), r,
                            alpha / (float)r, Y, y_dtype != QLORA_F32, T_save,
                            static_cast<char*>(ws), L, compute_dtype == QLORA_F16, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_t* W, const void* X, int64_t M, const void* A,
                                      const void* B, int32_t r, float alpha, void* Y, qlora_dtype y_dtype,
                                      float* T_save, void* stream) {
  const char* fn = "qlora_linear_fwd_noalloc";
  qlora_status st = check_fwd_args(fn, W, X, M, A, B, r, Y, y_dtype, T_save, QLORA_BF16);
  if (st != QLORA_OK) return st;
  // (splits of the GEMM's reduction are limited to what fits the array)
  const qnf4::FwdLayout L = qnf4::fwd_layout(M, W->n_rows, W->n_cols, r, kStaticScratchBytes);
  if (L.total > kStaticScratchBytes)
    return fail(QLORA_ERR_WORKSPACE_TOO_SMALL,
                "%s: this call needs %zu bytes of scratch; the static scratch holds %zu (use qlora_linear_fwd "
                "with a workspace)",
                fn, L.total, kStaticScratchBytes);
  if (M == 0) return ok();
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_status(fn, e);
  return hip_status(fn, qnf4::launch_forward(view(W), static_cast<const uint16_t*>(X), M,
                                             static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), r,
                                             alpha / (float)r, Y, y_dtype != QLORA_F32, T_save,
                                             static_cast<char*>(ws), L, false, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_linear_bwd(const qlora_nf4_t* W, const void* X, const void* dY, int64_t M,
                              const void* A, const void* B, int32_t r, float alpha,
                              const float* T_saved, void* dX, qlora_dtype dx_dtype, float* dA,
                              float* dB, void* ws, size_t ws_bytes, void* stream) {
  return qlora_linear_bwd_ex(W, X, dY, M, A, B, r, alpha, T_saved, dX, dx_dtype, dA, dB, ws, ws_bytes, QLORA_BF16,
                             stream);
}

qlora_status qlora_linear_bwd_ex(const qlora_nf4_t* W, const void* X, const void* dY, int64_t M,
                                 const void* A, const void* B, int32_t r, float alpha,
                                 const float* T_saved, void* dX, qlora_dtype dx_dtype, float* dA,
                                 float* dB, void* ws, size_t ws_bytes, qlora_dtype compute_dtype,
                                 void* stream) {
  const char* fn = "qlora_linear_bwd";
  qlora_status st = check_tensor(fn, W);
  if (st != QLORA_OK) return st;
  if (compute_dtype != QLORA_BF16 && compute_dtype != QLORA_F16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: compute_dtype=%d (BF16 or F16)", fn, compute_dtype);
  if ((st = check_rank(fn, r)) != QLORA_OK) return st;
  if (M < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: M=%lld < 0", fn, (long long)M);
  if ((st = check_linear_limits(fn, M, W->n_rows, W->n_cols, r)) != QLORA_OK) return st;
  if (dx_dtype != QLORA_F32 && dx_dtype != compute_dtype)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: dx_dtype=%d (F32 or the compute dtype)", fn, dx_dtype);
  CHECK_PTR(A);
  CHECK_PTR(B);
  CHECK_PTR(dA);
  CHECK_PTR(dB);
  if (M > 0) {
    CHECK_PTR(X);
    CHECK_PTR(dY);
    CHECK_PTR(dX);
  }
  CHECK_OPT_PTR(T_saved);
  const qnf4::BwdLayout L = qnf4::bwd_layout(M, W->n_rows, W->n_cols, r);
  if (ws_bytes < L.total)
    return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", fn, ws_bytes,
                L.total);
  CHECK_PTR(ws);
  return hip_status(fn, qnf4::launch_backward(
                            view(W), static_cast<const uint16_t*>(X),
                            static_cast<const uint16_t*>(dY), M, static_cast<const uint16_t*>(A),
                            static_cast<const uint16_t*>(B), r, alpha / (float)r, T_saved, dX,
                            dx_dtype != QLORA_F32, dA, dB, static_cast<char*>(ws), L, compute_dtype == QLORA_F16,
                            static_cast<hipStream_t>(stream)));
}

qlora_status qlora_adamw_step(const qlora_adamw_tensor_t* tensors, int32_t count,
                              qlora_dtype param_dtype, float lr, float beta1, float beta2, float eps,
                              float weight_decay, int64_t step, void* stream) {
  const char* fn = "qlora_adamw_step";
  if (tensors == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: tensors is NULL", fn);
  if (count < 1 || count > QLORA_ADAMW_MAX_TENSORS)
    return fail(QLORA_ERR_INVALID_ARG, "%s: count=%d outside [1, %d]", fn, count, QLORA_ADAMW_MAX_TENSORS);
  if (param_dtype != QLORA_F32 && param_dtype != QLORA_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: param_dtype=%d", fn, param_dtype);
  if (step < 1) return fail(QLORA_ERR_INVALID_ARG, "%s: step=%lld < 1", fn, (long long)step);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(QLORA_ERR_INVALID_ARG, "%s: betas (%g, %g) outside [0, 1)", fn, beta1, beta2);
  if (!(eps > 0.0f) || !(eps < INFINITY))
    return fail(QLORA_ERR_INVALID_ARG, "%s: eps=%g must be positive and finite", fn, eps);
  if (!(lr >= 0.0f && lr < INFINITY) || !(weight_decay >= 0.0f && weight_decay < INFINITY))
    return fail(QLORA_ERR_INVALID_ARG, "%s: lr=%g, weight_decay=%g must be finite and >= 0", fn, lr,
                weight_decay);
  qnf4::AdamwArgs a{};
  a.count = count;
  uint64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    const qlora_adamw_tensor_t& t = tensors[i];
    if (t.n < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: tensors[%d].n=%lld < 0", fn, i, (long long)t.n);
    if (t.n > 0) {
      const void* param = t.param;
      const void* grad = t.grad;
      const void* exp_avg = t.exp_avg;
      const void* exp_avg_sq = t.exp_avg_sq;
      CHECK_PTR(param);
      CHECK_PTR(grad);
      CHECK_PTR(exp_avg);
      CHECK_PTR(exp_avg_sq);
    }
    blocks += qnf4::adamw_blocks(t.n);
    a.t[i] = qnf4::AdamwTensor{t.param, t.grad, t.exp_avg, t.exp_avg_sq, t.n};
  }
  if (blocks > 0x7fffffffu) return fail(QLORA_ERR_INVALID_ARG, "%s: too many elements", fn);
  return hip_status(fn, qnf4::launch_adamw(a, param_dtype == QLORA_BF16, lr, beta1, beta2, eps,
                                           weight_decay, step, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_merge_lora(const qlora_nf4_t* W, const void* A, const void* B, int32_t r, float alpha,
                              void* out, qlora_dtype out_dtype, void* stream) {
  const char* fn = "qlora_merge_lora";
  qlora_status st = check_tensor(fn, W);
  if (st != QLORA_OK) return st;
  if ((st = check_rank(fn, r)) != QLORA_OK) return st;
  if (out_dtype != QLORA_BF16 && out_dtype != QLORA_F16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: out_dtype=%d (expected BF16 or F16)", fn, out_dtype);
  const int64_t N = W->n_rows, K = W->n_cols;
  if (N > (int64_t(1) << 31) / K || (int64_t)r * K > (int64_t(1) << 29) || N * r > (int64_t(1) << 29))
    return fail(QLORA_ERR_INVALID_ARG, "%s: N*K, r*K or N*r too large", fn);
  CHECK_PTR(A);
  CHECK_PTR(B);
  CHECK_PTR(out);
  return hip_status(fn, qnf4::launch_merge(view(W), static_cast<const uint16_t*>(A),
                                           static_cast<const uint16_t*>(B), r, alpha / (float)r,
                                           static_cast<uint16_t*>(out), out_dtype == QLORA_F16,
                                           static_cast<hipStream_t>(stream)));
}

namespace {

qlora_status check_qtensor(const char* fn, const qlora_qtensor_t* q) {
  if (q == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: tensor descriptor is NULL", fn);
  qlora_status st = check_shape(fn, q->n_rows, q->n_cols);
  if (st != QLORA_OK) return st;
  if (q->format != QLORA_FMT_NF4 && q->format != QLORA_FMT_INT4 && q->format != QLORA_FMT_INT8)
    return fail(QLORA_ERR_INVALID_ARG, "%s: format=%d", fn, q->format);
  const uint8_t* codes = q->codes;
  const float* absmax = q->absmax;
  CHECK_PTR(codes);
  CHECK_PTR(absmax);
  return QLORA_OK;
}

}  // namespace

qlora_status qlora_quantize_format(const void* W, qlora_dtype w_dtype, int64_t N, int64_t K,
                                   qlora_qtensor_t* out, void* stream) {
  const char* fn = "qlora_quantize_format";
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: w_dtype=%d (expected F32 or BF16)", fn, w_dtype);
  qlora_status st = check_shape(fn, N, K);
  if (st != QLORA_OK) return st;
  CHECK_PTR(W);
  if ((st = check_qtensor(fn, out)) != QLORA_OK) return st;
  if (out->n_rows != N || out->n_cols != K)
    return fail(QLORA_ERR_INVALID_ARG, "%s: descriptor shape %lldx%lld != %lldx%lld", fn,
                (long long)out->n_rows, (long long)out->n_cols, (long long)N, (long long)K);
  return hip_status(fn, qnf4::launch_format_quantize(W, w_dtype == QLORA_BF16, N, K, out->format, out->codes,
                                                     out->absmax, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_dequantize_format(const qlora_qtensor_t* q, void* out, qlora_dtype out_dtype,
                                     void* stream) {
  const char* fn = "qlora_dequantize_format";
  qlora_status st = check_qtensor(fn, q);
  if (st != QLORA_OK) return st;
  if (out_dtype != QLORA_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: out_dtype=%d (only BF16)", fn, out_dtype);
  CHECK_PTR(out);
  return hip_status(fn, qnf4::launch_format_dequantize(q->codes, q->absmax, q->format, q->n_rows, q->n_cols,
                                                       static_cast<uint16_t*>(out),
                                                       static_cast<hipStream_t>(stream)));
}

qlora_status qlora_gemv_format(const qlora_qtensor_t* q, const void* X, int64_t M, void* Y,
                               qlora_dtype y_dtype, void* stream) {
  const char* fn = "qlora_gemv_format";
  qlora_status st = check_qtensor(fn, q);
  if (st != QLORA_OK) return st;
  if (M < 0 || M > 16) return fail(QLORA_ERR_INVALID_ARG, "%s: M=%lld outside [0, 16]", fn, (long long)M);
  if (y_dtype != QLORA_F32 && y_dtype != QLORA_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: y_dtype=%d", fn, y_dtype);
  // one 16-row slice of codes must stay below 2^31 bytes (32-bit offsets)
  if (16 * q->n_cols > (int64_t(1) << 30)) return fail(QLORA_ERR_INVALID_ARG, "%s: K too large", fn);
  if (M > 0) {
    CHECK_PTR(X);
    CHECK_PTR(Y);
  }
  return hip_status(fn, qnf4::launch_format_gemv(q->codes, q->absmax, q->format, q->n_rows, q->n_cols,
                                                 static_cast<const uint16_t*>(X), M, Y, y_dtype == QLORA_BF16,
                                                 static_cast<hipStream_t>(stream)));
}

qlora_status qlora_time_next_launch(int32_t kernel_id, void* start_event, void* stop_event) {
  const char* fn = "qlora_time_next_launch";
  if (kernel_id < QLORA_KERNEL_NONE || kernel_id > QLORA_KERNEL_FORMAT_GEMV)
    return fail(QLORA_ERR_INVALID_ARG, "%s: unknown kernel id %d", fn, kernel_id);
  if (kernel_id != QLORA_KERNEL_NONE && (start_event == nullptr || stop_event == nullptr))
    return fail(QLORA_ERR_INVALID_ARG, "%s: NULL event", fn);
  qnf4::TimingHook& h = qnf4::timing_hook();
  h.kernel = kernel_id;
  h.start = static_cast<hipEvent_t>(start_event);
  h.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

qlora_status qlora_bench_mfma_peak(int64_t iters, float* sink, int64_t* flop, void* stream) {
  const char* fn = "qlora_bench_mfma_peak";
  if (iters < 1 || iters > (int64_t(1) << 30)) return fail(QLORA_ERR_INVALID_ARG, "%s: iters=%lld", fn, (long long)iters);
  CHECK_PTR(sink);
  if (flop == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: flop is NULL", fn);
  *flop = qnf4::mfma_peak_flop(iters);
  return hip_status(fn, qnf4::launch_mfma_peak(iters, sink, static_cast<hipStream_t>(stream)));
}

qlora_status qlora_bench_wall_clock_khz(int32_t* khz) {
  const char* fn = "qlora_bench_wall_clock_khz";
  if (khz == nullptr) return fail(QLORA_ERR_INVALID_ARG, "%s: khz is NULL", fn);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return hip_status(fn, e);
}

qlora_status qlora_bench_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  const char* fn = "qlora_bench_copy";
  CHECK_PTR(src);
  CHECK_PTR(dst);
  if (bytes <= 0 || bytes % 16 != 0)
    return fail(QLORA_ERR_INVALID_ARG, "%s: bytes=%lld must be a positive multiple of 16", fn, (long long)bytes);
  return hip_status(fn, qnf4::launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

void qlora_nf4_codebook(float* out16) {
  if (out16 == nullptr) return;
  std::memcpy(out16, qnf4::codebook().q, 16 * sizeof(float));
}

const char* qlora_status_string(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case QLORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QLORA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* qlora_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
