// Internal interface between the C-ABI layer (capi.hip) and the kernel
// launchers.  Launchers assume validated arguments and only enqueue work; they
// return the status of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace qnf4 {

const Codebook& codebook();

// One-shot timing request of the calling thread (see qlora_time_next_launch).
struct TimingHook {
  int kernel;
  hipEvent_t start, stop;
};
TimingHook& timing_hook();

// Launches kernel `k`.  If the calling thread asked to time the next launch
// of `kernel_id`, the launch carries the caller's start/stop events, which
// the runtime records around the dispatch itself (tighter than recording the
// events on the stream before and after), and the request is cleared.
template <typename F, typename... Args>
hipError_t timed_launch_shm(int kernel_id, F k, dim3 grid, dim3 block, size_t shm, hipStream_t st, Args... args) {
  TimingHook& h = timing_hook();
  if (h.kernel == kernel_id) {
    h.kernel = 0;
    hipExtLaunchKernelGGL(k, grid, block, shm, st, h.start, h.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(k, grid, block, shm, st, args...);
  }
  return hipGetLastError();
}
template <typename F, typename... Args>
hipError_t timed_launch(int kernel_id, F k, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  return timed_launch_shm(kernel_id, k, grid, block, 0, st, args...);
}
enum { kKernFwdGemm = 1, kKernDxGemm = 2, kKernGemv = 3, kKernQuantize = 4, kKernAdamw = 5, kKernMerge = 6, kKernFormatGemv = 7 };

// Round `x` up to a multiple of `a`.
constexpr int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Padded LoRA rank: the hi/lo split of s·T (and s·U) occupies [M, 2*Rp] bf16
// with hi in columns [0, r), lo in [Rp, Rp + r), zeros elsewhere.
inline int64_t lora_rp(int32_t r) { return round_up(r, 32); }

// Quantize ---------------------------------------------------------------
struct QuantLayout {
  int64_t nb, ng, chunks;   // blocks, DQ groups, 256-block chunks
  int64_t lvl_len[8];       // lengths of the tree-reduction levels (0-terminated)
  size_t off_absmax, off_partial, off_lvl_a, off_lvl_b, total;
};
QuantLayout quant_layout(int64_t N, int64_t K);

hipError_t launch_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* e, float* s, float* mu, char* ws, const QuantLayout& L,
                           hipStream_t st);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* e, const float* s,
                             const float* mu, int64_t N, int64_t K, uint16_t* out, bool f16,
                             hipStream_t st);

// Shared view of a quantized weight for the GEMM kernels.
struct Nf4View {
  const uint8_t* codes;
  const uint8_t* e;
  const float* s;
  const float* mu;
  int64_t N, K;
};

// LoRA side products -------------------------------------------------------
// Stream-K split of a product (see lora.hip): `tiles` output tiles, ut
// units per tile, U units in all over G workgroups; a tile collects at most
// cmax partial sums.
constexpr uint32_t kSkWorkgroups = 256;  // one per compute unit of an MI355X
struct SkPlan {
  int64_t tiles;
  uint32_t ut, U, G;
  int cmax, jt;
};
// T = X·Aᵀ, U = dY·B: reduction over Kred for M rows, 64x64 tiles
SkPlan rowred_plan(int64_t M, int64_t Kred, int64_t Rp);
// dA, dB: reduction over Mred for Pn columns, 128x64 tiles, on at most
// gmax workgroups.  The two run in one launch: dA on colred_split(K, N, Rp)
// of the 256 workgroups, dB on the rest.
SkPlan colred_plan(int64_t Mred, int64_t Pn, int64_t Rp, uint32_t gmax);
uint32_t colred_split(int64_t K, int64_t N, int64_t Rp);
size_t rowred_partial_bytes(const SkPlan& p);
size_t colred_partial_bytes(const SkPlan& p);
// Columns of the transposed bf16 splits [2Rp, Mp]: M rounded up to 64.
int64_t lora_mp(int64_t M);
// Partial tiles of Σ_k L[m][k]·R[j][k] (rows of R past rrows read as zero).
hipError_t launch_rowred(const uint16_t* L, int64_t M, int64_t Kred, int64_t ldl, const uint16_t* R,
                         int64_t rrows, int64_t ldr, const SkPlan& p, float* P, bool f16, hipStream_t st);
// Sums them → optional fp32 T [M, r], the hi/lo split of scale·T [M, 2Rp]
// and optionally its transpose [2Rp, Mp]; if B2 is given, the same launch
// also writes B2 [N, 2Rp] = [B | B] zero-padded (the forward GEMM's operand).
hipError_t launch_rowred_finish(const float* P, const SkPlan& p, int64_t M, int32_t r, int64_t Rp,
                                float scale, float* T, uint16_t* out, uint16_t* outT, const uint16_t* B,
                                int64_t N, uint16_t* B2, bool f16, hipStream_t st);
// Partial tiles of Σ_m L[m][p]·(S[j][m] + S[Rp + j][m]).
struct ColredJob {  // one adapter gradient's reduction (see lora.hip)
  const uint16_t* L;
  int64_t Mred, ldl;
  const uint16_t* S;
  int64_t lds, Rp;
  int jt;
  uint32_t ut, U, G;
  int cmax;
  float* P;
};
hipError_t launch_colred(const ColredJob& a, const ColredJob& b, bool f16, hipStream_t st);
// Sums them → out [Pn, r], or out [r, Pn] when transposed.
struct ColredFinishJob {
  const float* P;
  int jt;
  uint32_t ut, U, G;
  int cmax;
  int64_t Pn, tiles;
  int transpose;
  float* out;
};
hipError_t launch_colred_finish(const ColredFinishJob& a, const ColredFinishJob& b, int32_t r, hipStream_t st);
// The backward pass's operand copies, one launch: if T is non-null, sT
// [M, 2Rp] and sTT [2Rp, Mp] from the saved T; BT [Rp, round_up(N, 64)] =
// Bᵀ zero-padded; AT2 [K, 2Rp] = [Aᵀ | Aᵀ] zero-padded.
hipError_t launch_bwd_prep(const float* T, int64_t M, int32_t r, int64_t Rp, float scale, uint16_t* sT,
                           uint16_t* sTT, const uint16_t* B, int64_t N, uint16_t* BT, const uint16_t* A,
                           int64_t K, uint16_t* AT2, bool f16, hipStream_t st);
hipError_t launch_zero(float* a, int64_t n, hipStream_t st);

// Dequant-GEMV (M <= 16): bytes of the partial tiles of T = X·Aᵀ.
size_t gemv_partial_bytes(int64_t K, int32_t r);

// Forward ------------------------------------------------------------------
struct FwdLayout {
  // fp32 T [M, r] (if not saved by the caller), bf16 sT [M, 2Rp], bf16 B2
  // [N, 2Rp], one fp32 partial-sum area: first the partial sums of T over
  // the reduction slices, then (splits > 1) the GEMM's split partials
  // [splits, M, N]
  size_t off_T, off_sT, off_B2, off_P, total;
  SkPlan pT;
  int splits;
};
// cap: the most bytes the layout may take; the GEMM's reduction splits are
// reduced until it fits (the layout may still exceed cap without splits).
FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, size_t cap = SIZE_MAX);
// The largest fwd_layout(M, ...).total over M in [0, M_max].
size_t fwd_ws_bytes_max(int64_t M_max, int64_t N, int64_t K, int32_t r);

hipError_t launch_forward(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                          const uint16_t* B, int32_t r, float scale, void* Y, bool y16,
                          float* T, char* ws, const FwdLayout& L, bool f16, hipStream_t st);

// Backward -----------------------------------------------------------------
struct BwdLayout {
  // bf16 sT, sU [M, 2Rp] and their transposes sTT, sUT [2Rp, Mp]; bf16 BT
  // [Rp, round_up(N, 64)]; bf16 AT2 [K, 2Rp]; one fp32 partial-sum area
  // reused by the T, U, dA and dB reductions and (splits > 1) the dX GEMM's
  // split partials [splits, M, K]
  size_t off_sT, off_sTT, off_sU, off_sUT, off_BT, off_AT2, off_P, total;
  SkPlan pT, pU, pA, pB;
  int splits;
};
BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r);
// The largest bwd_layout(M, ...).total over M in [0, M_max].
size_t bwd_ws_bytes_max(int64_t M_max, int64_t N, int64_t K, int32_t r);

hipError_t launch_backward(const Nf4View& W, const uint16_t* X, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                           const float* T_saved, void* dX, bool dx16, float* dA, float* dB,
                           char* ws, const BwdLayout& L, bool f16, hipStream_t st);

// AdamW on the LoRA parameters ---------------------------------------------
constexpr int kAdamwMaxTensors = 8;
struct AdamwTensor {
  void* p;         // parameter, bf16 or fp32
  const float* g;  // gradient
  float* m;        // first moment
  float* v;        // second moment
  int64_t n;
};
struct AdamwArgs {
  AdamwTensor t[kAdamwMaxTensors];
  uint32_t block0[kAdamwMaxTensors + 1];  // first block of each tensor (set by the launcher)
  int count;
};
uint32_t adamw_blocks(int64_t n);
hipError_t launch_adamw(AdamwArgs a, bool param_bf16, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int64_t step, hipStream_t st);

// LoRA merge -----------------------------------------------------------------
hipError_t launch_merge(const Nf4View& W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                        uint16_t* out, bool out_f16, hipStream_t st);

// Comparison formats ------------------------------------------------------------
// fmt: 1 NF4 (double quantization off), 2 absmax INT4, 3 absmax INT8
hipError_t launch_format_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, int fmt, uint8_t* codes,
                                  float* absmax, hipStream_t st);
hipError_t launch_format_dequantize(const uint8_t* codes, const float* absmax, int fmt, int64_t N, int64_t K,
                                    uint16_t* out, hipStream_t st);
hipError_t launch_format_gemv(const uint8_t* codes, const float* absmax, int fmt, int64_t N, int64_t K,
                              const uint16_t* X, int64_t M, void* Y, bool y_bf16, hipStream_t st);

// Benchmark instrumentation -------------------------------------------------
constexpr int kPeakWorkgroups = 2048;  // 8 waves per compute unit of an MI355X
int64_t mfma_peak_flop(int64_t iters);
hipError_t launch_mfma_peak(int64_t iters, float* sink, hipStream_t st);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);

}  // namespace qnf4
