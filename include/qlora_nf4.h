/*
 * qlora_nf4.h -- C ABI of the NF4 QLoRA linear-layer library for MI355X
 * (gfx950).  Every entry point is extern "C", takes plain pointers and sizes,
 * and no type from any framework.
 *
 * Page tags used in the citations (see the oracle package for the full list):
 *   P1 "QLoRA 的原理是什么？4-bit 量化权重真的参与训练吗？" (offer.aigcbaba.com)
 *   P2 review of "QLoRA: Efficient Finetuning of Quantized LLMs" (ainexis.cn)
 *   P3 "Ch.09 QLoRA 与量化：缩得更小再微调" (mdooai.com)
 *   P4 "M5 · PEFT (LoRA / QLoRA / Prefix Tuning)" science-depth card (airsota.com)
 *
 * Conventions shared by all entry points
 *   - Pointers named "device" are HIP device pointers owned by the caller; the
 *     library never allocates, frees or keeps them.  Host pointers are read or
 *     written before the call returns.
 *   - Device pointers must be 16-byte aligned.  Tensors are dense row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no call synchronizes the stream.  Results are valid once
 *     the stream has reached the enqueued work.
 *   - Every argument is validated on the host before any HIP call is made; on
 *     an invalid argument nothing is enqueued and an error status is returned.
 *     qlora_last_error() then gives a text for the failing check (per thread).
 *   - Calls are stateless and thread-safe.  Two calls that share output or
 *     workspace memory must be ordered by the caller (same stream, or events).
 *   - Floating-point results for non-finite inputs are unspecified.
 *   - Shapes: W is [N, K] = [out_features, in_features] with K % 64 == 0 and
 *     N % 8 == 0; X is [M, K]; Y and dY are [M, N]; LoRA A is [r, K], B is
 *     [N, r], 1 <= r <= 256; s = alpha / r.  M may be 0.
 *   - Limits of one linear pass (forward or backward), from the kernels'
 *     32-bit buffer offsets: N*K/2 < 2^31 (packed codes),
 *     M*max(N, K) < 2^30 (activations and gradients of one call) and
 *     2*Rp*round_up(M, 64)*2 < 2^31 with Rp = round_up(r, 32); beyond them
 *     the call returns QLORA_ERR_INVALID_ARG.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qlora_status;
#define QLORA_OK 0
#define QLORA_ERR_INVALID_ARG 1        /* null pointer, bad size, misalignment */
#define QLORA_ERR_UNSUPPORTED_DTYPE 2  /* dtype not accepted by this entry point */
#define QLORA_ERR_WORKSPACE_TOO_SMALL 3
#define QLORA_ERR_HIP 4                /* a HIP launch or runtime call failed */

typedef int32_t qlora_dtype;
#define QLORA_F32 0
#define QLORA_BF16 1
#define QLORA_F16 2  /* IEEE binary16: the alternative compute format (the *_ex
                        entry points), dequantize and merge outputs */

/* One NF4 + double-quantized weight (P4 §三 English derivation; P1 §二).
 * All four arrays are device memory:
 *   codes        uint8[N*K/2]: flattened element i is the low nibble of byte
 *                i/2 if i is even, the high nibble if i is odd;
 *   absmax_e4m3  uint8[N*K/64]: OCP FP8 E4M3 code of block b's mean-centred,
 *                group-scaled absmax;
 *   dq_scale     float[ceil(N*K/64/256)]: one fp32 scale per 256 constants;
 *   dq_mean      float[1]: the tensor's mean of all block absmax values. */
typedef struct {
  int64_t n_rows; /* N = out_features */
  int64_t n_cols; /* K = in_features, a multiple of 64 */
  uint8_t* codes;
  uint8_t* absmax_e4m3;
  float* dq_scale;
  float* dq_mean;
} qlora_nf4_t;

/* Byte counts for one layer.  Workspace sizes cover every M in [0, M_max]. */
typedef struct {
  size_t codes_bytes;       /* N*K/2 */
  size_t absmax_bytes;      /* N*K/64 */
  size_t scale_bytes;       /* 4*ceil(N*K/64/256) */
  size_t mean_bytes;        /* 4 */
  size_t quantize_ws_bytes; /* workspace of qlora_nf4_quantize */
  size_t fwd_ws_bytes;      /* workspace of qlora_linear_fwd for M <= M_max */
  size_t bwd_ws_bytes;      /* workspace of qlora_linear_bwd for M <= M_max */
} qlora_sizes_t;

/* Host-only size query.  Errors: N, K, r out of range (see conventions),
 * M_max < 0, out == NULL. */
qlora_status qlora_nf4_sizes(int64_t N, int64_t K, int64_t M_max, int32_t r,
                             qlora_sizes_t* out);

/* Blockwise NF4 quantization with double quantization of the constants.
 * (P4 §三 English derivation: W_norm = W / max|W_block| over B = 64 elements,
 * code = the nearest of 16 standard-normal-quantile levels that include an
 * exact zero; the fp32 block constants are quantized to an 8-bit float with a
 * second-level block of 256.  P4 §二: this saves about 0.37 bit/param.)
 *   W        device, [N, K] fp32 (w_dtype QLORA_F32) or bf16 (QLORA_BF16);
 *   out      host struct whose four device arrays receive the result;
 *            out->n_rows/n_cols must equal N/K;
 *   ws       device workspace of at least qlora_nf4_sizes().quantize_ws_bytes.
 * Per block b: c_b = max|w|; x = fl32(w / c_b) (one correctly rounded
 * division); code = argmin_j |x - q_j| with ties to the lower index; c_b == 0
 * gives code 7 (the zero level).  mu = fl32(S / nb) with S the fp64 balanced
 * pairwise sum of all c_b; per group g of 256 constants
 * s_g = fl32(max|fl32(c_b - mu)| / 448) and e_b = E4M3(fl32(d_b / s_g)) with
 * round-to-nearest-even and saturation at 448 (all zero if s_g == 0). */
qlora_status qlora_nf4_quantize(const void* W, qlora_dtype w_dtype, int64_t N,
                                int64_t K, const qlora_nf4_t* out, void* ws,
                                size_t ws_bytes, void* stream);

/* Dequantize to bf16 (P1 §七: the 4-bit base is dequantized block by block to
 * BF16 before the matmul; P4 §四 ①: Ŵ = Dequant(W^NF4)·c).
 *   q        host struct describing the quantized weight (device arrays);
 *   out      device, [N, K] bf16 (out_dtype QLORA_BF16) or fp16 (QLORA_F16,
 *            the same product rounded into binary16).
 * ŵ = RNE_bf16(fl32(q[code] * c')) with
 * c' = fl32(fl32(dec(e) * s_g) + mu); bit-exact, signed zeros kept. */
qlora_status qlora_dequantize(const qlora_nf4_t* q, void* out,
                              qlora_dtype out_dtype, void* stream);

/* QLoRA linear forward (P1 §七 dataflow figure; P3 公式导读 3: a frozen wide
 * path plus a trainable low-rank path, summed):
 *   Y = X·Ŵᵀ + (alpha/r)·(X·Aᵀ)·Bᵀ
 *   W        host struct of the quantized weight [N, K];
 *   X        device bf16 [M, K];  A device bf16 [r, K];  B device bf16 [N, r];
 *   Y        device [M, N], bf16 (y_dtype QLORA_BF16) or fp32 (QLORA_F32);
 *   T_save   device fp32 [M, r] receiving T = X·Aᵀ for the backward pass, or
 *            NULL (T then lives in the workspace only);
 *   ws       device workspace of at least qlora_nf4_sizes(..., M_max >= M,
 *            r).fwd_ws_bytes.
 * fp32 accumulation; M <= 16 takes a dequant-GEMV path, larger M a
 * dequant-in-tile MFMA GEMM.  No bias, no dropout.  Y must not alias inputs. */
qlora_status qlora_linear_fwd(const qlora_nf4_t* W, const void* X, int64_t M,
                              const void* A, const void* B, int32_t r,
                              float alpha, void* Y, qlora_dtype y_dtype,
                              float* T_save, void* ws, size_t ws_bytes,
                              void* stream);

/* QLoRA linear backward (P1 简化版 and §七, P2 §4.4: the gradient passes
 * through the dequantized frozen weight into the LoRA parameters only; the
 * 4-bit codes and constants are never updated, so no weight gradient exists).
 * With U = dY·B:
 *   dX = dY·Ŵ + s·U·A;   dA = s·Uᵀ·X;   dB = s·dYᵀ·T,  T = X·Aᵀ.
 *   dY       device bf16 [M, N];  X, A, B as in the forward pass;
 *   T_saved  device fp32 [M, r] from qlora_linear_fwd, or NULL to recompute;
 *   dX       device [M, K], bf16 or fp32 (dx_dtype);
 *   dA       device fp32 [r, K] (overwritten, not accumulated);
 *   dB       device fp32 [N, r] (overwritten, not accumulated);
 *   ws       device workspace of at least .bwd_ws_bytes.
 * With M == 0, dA and dB are set to zero. */
qlora_status qlora_linear_bwd(const qlora_nf4_t* W, const void* X,
                              const void* dY, int64_t M, const void* A,
                              const void* B, int32_t r, float alpha,
                              const float* T_saved, void* dX,
                              qlora_dtype dx_dtype, float* dA, float* dB,
                              void* ws, size_t ws_bytes, void* stream);

/* The same two passes in either 16-bit compute format (P1 §四 and §七 name
 * FP16 beside BF16 as the precision the dequantized weight is multiplied in):
 * compute_dtype QLORA_BF16 (what qlora_linear_fwd / qlora_linear_bwd use) or
 * QLORA_F16.  X, dY, A and B are in the compute format; the weight is
 * dequantized into it (RNE16(fl32(q·c'))); the hi/lo splits of s·T and s·U are
 * pairs of that format; accumulation is fp32.  y_dtype / dx_dtype: QLORA_F32
 * or the compute format.  Everything else as above. */
qlora_status qlora_linear_fwd_ex(const qlora_nf4_t* W, const void* X, int64_t M,
                                 const void* A, const void* B, int32_t r,
                                 float alpha, void* Y, qlora_dtype y_dtype,
                                 float* T_save, void* ws, size_t ws_bytes,
                                 qlora_dtype compute_dtype, void* stream);
qlora_status qlora_linear_bwd_ex(const qlora_nf4_t* W, const void* X,
                                 const void* dY, int64_t M, const void* A,
                                 const void* B, int32_t r, float alpha,
                                 const float* T_saved, void* dX,
                                 qlora_dtype dx_dtype, float* dA, float* dB,
                                 void* ws, size_t ws_bytes,
                                 qlora_dtype compute_dtype, void* stream);

/* qlora_linear_fwd for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * forward pass (bf16 compute) without a workspace argument: its scratch
 * memory (T, the hi/lo split of s·T, the [B | B] operand and the partial sums
 * of the split reductions) lives in a static 32 MiB device array of the
 * library, one per GPU, held until the process ends.  The library allocates
 * and frees nothing.
 *   Arguments as qlora_linear_fwd; the calling thread's current device must
 *   be the device of `stream`.
 *   A call that needs more than 32 MiB of scratch (the fwd_ws_bytes that
 *   qlora_nf4_sizes reports for its M) returns QLORA_ERR_WORKSPACE_TOO_SMALL
 *   before any HIP call; every linear of the 7B and 65B shapes fits up to
 *   8192 tokens at rank 64.
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 *   call's contents (nothing relies on them): calls that overlap on one GPU
 *   (other streams or host threads, unordered) race and give wrong results;
 *   the caller orders them. */
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_t* W, const void* X, int64_t M,
                                      const void* A, const void* B, int32_t r,
                                      float alpha, void* Y, qlora_dtype y_dtype,
                                      float* T_save, void* stream);

/* One tensor of LoRA parameters for qlora_adamw_step (all device memory,
 * 16-byte aligned when n > 0):
 *   param       n elements, bf16 or fp32 (the call's param_dtype), updated in
 *               place;
 *   grad        fp32 [n] (e.g. dA or dB of qlora_linear_bwd);
 *   exp_avg     fp32 [n], first moment, updated in place;
 *   exp_avg_sq  fp32 [n], second moment, updated in place. */
typedef struct {
  void* param;
  const float* grad;
  float* exp_avg;
  float* exp_avg_sq;
  int64_t n;
} qlora_adamw_tensor_t;
#define QLORA_ADAMW_MAX_TENSORS 8

/* One AdamW step on up to QLORA_ADAMW_MAX_TENSORS tensors in one launch.
 * (P1 §七 table: only the LoRA parameters are trained, optimizer state exists
 * only for them, in FP32; P4 §三 English derivation, item 3: a 32-bit AdamW
 * over the LoRA parameters; P4 §四 ④: the parameters are kept in BF16.)
 *   tensors      host array of `count` descriptors, 1 <= count <= 8;
 *   param_dtype  QLORA_BF16 or QLORA_F32 for every tensor's param;
 *   step         the 1-based step number t (bias corrections 1 - beta^t);
 *   0 <= beta1, beta2 < 1, eps > 0, lr >= 0, weight_decay >= 0, all finite.
 * With decay = fl(1 - fl(lr*wd)), omb = fl(1 - beta), bc = fl32(1 - beta^t)
 * (power in fp64), sbc2 = fl(sqrt(bc2)) and step_size = fl(lr / bc1), each
 * element takes, one binary32 rounding per operation and no fused
 * multiply-add: p = fl(p*decay); m = fl(fl(b1*m) + fl(omb1*g));
 * v = fl(fl(b2*v) + fl(fl(omb2*g)*g)); d = fl(fl(sqrt(v)/sbc2) + eps);
 * p = fl(p - fl(step_size * fl(m/d))).  A bf16 parameter is widened exactly
 * before and rounded to nearest-even after.  Tensors must not overlap. */
qlora_status qlora_adamw_step(const qlora_adamw_tensor_t* tensors, int32_t count,
                              qlora_dtype param_dtype, float lr, float beta1,
                              float beta2, float eps, float weight_decay,
                              int64_t step, void* stream);

/* The LoRA adapter merged into the dequantized weight, for serving (P5,
 * follow-up 1: the fine-tuned model converted once to 16 bits with the LoRA
 * weights merged into the dequantized weight; P1 §七 dataflow figure: the
 * layer is X·(Ŵ + s·B·A)ᵀ; P1 §五: merging and re-quantizing can bring the
 * quantization error back -- re-quantize by passing a bf16 result to
 * qlora_nf4_quantize):
 *   W_m[n][k] = RND(fl32(ŵ[n][k] + fl32(s · Σ_j B[n][j]·A[j][k]))),
 * with ŵ the dequantized bf16 weight of qlora_dequantize, s = fl32(alpha/r),
 * the rank-r sum accumulated in fp32 and RND the round to nearest even into
 * out_dtype.  Against the exact sum rounded once to out_dtype the result is
 * within one unit in the last place.
 *   W          NF4 weight [N, K];
 *   A          device bf16 [r, K];  B  device bf16 [N, r];  1 <= r <= 256;
 *   out        device [N, K], QLORA_BF16 or QLORA_F16 (out_dtype);
 * Limits: N*K <= 2^31, r*K <= 2^29, N*r <= 2^29.  No workspace. */
qlora_status qlora_merge_lora(const qlora_nf4_t* W, const void* A,
                              const void* B, int32_t r, float alpha,
                              void* out, qlora_dtype out_dtype, void* stream);

/* Comparison formats of the frozen weight (a second workload: P4 §三, NF4's
 * fp32 block constants before double quantization; P2 §4.1 and P4 trade-off
 * ②, uniform 4-bit integers against NF4; P3 公式导读 2, absmax INT8).  Each
 * keeps one fp32 absmax c per 64-block of the flattened weight and no double
 * quantization; w' = RNE_bf16(fl32(L[code]·c)):
 *   QLORA_FMT_NF4   NF4 codes (those of qlora_nf4_quantize), packed 2 per
 *                   byte; L = the NF4 levels;
 *   QLORA_FMT_INT4  k = round(fl32(w · fl32(7/c))), halves away from zero,
 *                   k in [-7, 7], stored as the nibble k + 8, packed 2 per
 *                   byte; L = fl32(k/7);
 *   QLORA_FMT_INT8  the same with 127, one byte per weight (two's complement);
 *                   L = fl32(k/127).
 * A block of zeros gets the zero code.  codes: N*K/2 bytes (NF4, INT4) or
 * N*K bytes (INT8); absmax: N*K/64 floats; both device memory. */
#define QLORA_FMT_NF4 1
#define QLORA_FMT_INT4 2
#define QLORA_FMT_INT8 3
typedef struct {
  int64_t n_rows;    /* N */
  int64_t n_cols;    /* K, a multiple of 64 */
  int32_t format;    /* QLORA_FMT_* */
  uint8_t* codes;
  float* absmax;
} qlora_qtensor_t;

/* Quantize W [N, K] (fp32 or bf16, device) into `out`'s format; no
 * workspace.  Errors as qlora_nf4_quantize, plus an unknown format. */
qlora_status qlora_quantize_format(const void* W, qlora_dtype w_dtype,
                                   int64_t N, int64_t K, qlora_qtensor_t* out,
                                   void* stream);

/* w' of every weight into out [N, K] bf16 (device; out_dtype QLORA_BF16). */
qlora_status qlora_dequantize_format(const qlora_qtensor_t* q, void* out,
                                     qlora_dtype out_dtype, void* stream);

/* The dequant-GEMV Y = X·Ŵᵀ for 0 <= M <= 16 tokens (no adapter): X device
 * bf16 [M, K]; Y device [M, N], bf16 or fp32 (y_dtype); fp32 accumulation.
 * Limits: codes and absmax of one 16-row slice below 2^31 bytes. */
qlora_status qlora_gemv_format(const qlora_qtensor_t* q, const void* X,
                               int64_t M, void* Y, qlora_dtype y_dtype,
                               void* stream);

/* Benchmark instrumentation.  The next launch of kernel `kernel_id` made by
 * the calling thread is bracketed by hipEventRecord(start_event) and
 * hipEventRecord(stop_event) on that launch's stream; then the request is
 * cleared (one-shot).  Both events are hipEvent_t handles created and owned by
 * the caller.  kernel_id: QLORA_KERNEL_NONE cancels a pending request.
 * Errors: unknown kernel id; a NULL event with a kernel id other than NONE. */
#define QLORA_KERNEL_NONE 0
#define QLORA_KERNEL_FWD_GEMM 1   /* dequant-in-tile forward GEMM (M > 16) */
#define QLORA_KERNEL_DX_GEMM 2    /* dequant-in-tile dX GEMM */
#define QLORA_KERNEL_GEMV 3       /* dequant-GEMV forward (M <= 16) */
#define QLORA_KERNEL_QUANTIZE 4   /* blockwise NF4 quantization kernel */
#define QLORA_KERNEL_ADAMW 5      /* AdamW step kernel */
#define QLORA_KERNEL_MERGE 6      /* LoRA merge kernel */
#define QLORA_KERNEL_FORMAT_GEMV 7 /* dequant-GEMV of the comparison formats */
qlora_status qlora_time_next_launch(int32_t kernel_id, void* start_event, void* stop_event);

/* Benchmark reference points (not part of the method).
 * qlora_bench_mfma_peak: 2048 workgroups of 4 waves issue `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 from registers; *flop receives the
 * dense bf16 FLOP the launch performs, so FLOP / the launch's time is the
 * MFMA rate the chip sustains.  sink: device array of 2056 floats, 8-byte
 * aligned; its first 2048 are written only in a case that does not occur;
 * the last 8 receive four uint64 values from the first lane of workgroup 0:
 * the shader clock counter before and after its loop, then the real-time
 * counter before and after (its rate: qlora_bench_wall_clock_khz).
 * 1 <= iters <= 2^30.
 * qlora_bench_wall_clock_khz: the current device's real-time counter rate
 * in kHz (hipDeviceAttributeWallClockRate).
 * qlora_bench_copy: a streaming copy of `bytes` (a positive multiple of 16)
 * from src to dst (device, 16-byte aligned, not overlapping): the HBM rate of
 * a plain read + write, and the calibration of the HBM byte counters. */
qlora_status qlora_bench_mfma_peak(int64_t iters, float* sink, int64_t* flop, void* stream);
qlora_status qlora_bench_copy(const void* src, void* dst, int64_t bytes, void* stream);
qlora_status qlora_bench_wall_clock_khz(int32_t* khz);

/* The 16 fp32 NF4 levels as the library computes them (host memory, 16
 * floats), ascending, index 7 = 0.  (P4 §三: levels at standard-normal
 * quantiles with equal probability mass, an exact zero, ends at ±1.) */
void qlora_nf4_codebook(float* out16);

/* Text for a status code, and the detail of the calling thread's last error. */
const char* qlora_status_string(qlora_status s);
const char* qlora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
