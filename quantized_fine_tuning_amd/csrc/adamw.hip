// AdamW step on the LoRA parameters, gfx950.
//
// P1 §七 (table of storage and compute precisions): only the LoRA parameters
// are trained and optimizer state exists only for them, in FP32.  P4 §三
// (English derivation, item 3): a 32-bit AdamW over the LoRA parameters.
// P4 §四 ④: the parameters themselves are kept in BF16.
//
// Per element, every operation one IEEE binary32 rounding, no fused
// multiply-add (the step constants come from the host):
//   p = fl(p * decay)
//   m = fl(fl(b1 * m) + fl(omb1 * g))
//   v = fl(fl(b2 * v) + fl(fl(omb2 * g) * g))
//   d = fl(fl(sqrt(v) / sbc2) + eps)
//   p = fl(p - fl(step_size * fl(m / d)))
// with a bf16 parameter widened exactly before and rounded to nearest-even
// after.  The step streams each element once: 24 bytes per parameter with a
// bf16 parameter (read 2 + 4 + 4 + 4, write 2 + 4 + 4), 28 with an fp32 one.
//
// One launch covers up to kAdamwMaxTensors tensors: the grid is the
// concatenation of the tensors' block ranges, each thread takes 4
// consecutive elements (16-byte loads of the fp32 arrays); the last,
// partial quadruple of a tensor goes element by element.
#include <cmath>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int kAdamwThreads = 256, kAdamwPerThread = 4;

struct Step {
  float b1, b2, eps, decay, omb1, omb2, sbc2, step_size;
};

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const Step& c) {
  p = __fmul_rn(p, c.decay);
  m = __fadd_rn(__fmul_rn(c.b1, m), __fmul_rn(c.omb1, g));
  v = __fadd_rn(__fmul_rn(c.b2, v), __fmul_rn(__fmul_rn(c.omb2, g), g));
  // (__builtin_sqrtf is the correctly rounded square root under
  // -fhip-fp32-correctly-rounded-divide-sqrt; __fsqrt_rn lowers to the bare
  // hardware instruction, which is not)
  const float d = __fadd_rn(__fdiv_rn(__builtin_sqrtf(v), c.sbc2), c.eps);
  p = __fsub_rn(p, __fmul_rn(c.step_size, __fdiv_rn(m, d)));
}

template <bool BF16>
__global__ __launch_bounds__(kAdamwThreads) void adamw_kernel(AdamwArgs a, Step c) {
  const uint32_t b = blockIdx.x;
  int t = 0;
#pragma unroll
  for (int i = 1; i < kAdamwMaxTensors; ++i) t += (i < a.count && b >= a.block0[i]) ? 1 : 0;
  const AdamwTensor x = a.t[t];
  const int64_t i0 = ((int64_t)(b - a.block0[t]) * kAdamwThreads + threadIdx.x) * kAdamwPerThread;
  if (i0 >= x.n) return;
  if (i0 + kAdamwPerThread <= x.n) {
    const f32x4_t g = *reinterpret_cast<const f32x4_t*>(x.g + i0);
    f32x4_t m = *reinterpret_cast<const f32x4_t*>(x.m + i0);
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(x.v + i0);
    float p[4];
    if constexpr (BF16) {
      const u32x2_t pb = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(x.p) + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = bf16_to_f32((uint16_t)(pb[e >> 1] >> (16 * (e & 1))));
    } else {
      const f32x4_t pf = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(x.p) + i0);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = pf[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float me = m[e], ve = v[e];
      adamw_one(p[e], g[e], me, ve, c);
      m[e] = me;
      v[e] = ve;
    }
    *reinterpret_cast<f32x4_t*>(x.m + i0) = m;
    *reinterpret_cast<f32x4_t*>(x.v + i0) = v;
    if constexpr (BF16) {
      u32x2_t pb;
      pb[0] = pack_bf16x2(p[0], p[1]);
      pb[1] = pack_bf16x2(p[2], p[3]);
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(x.p) + i0) = pb;
    } else {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(x.p) + i0) = f32x4_t{p[0], p[1], p[2], p[3]};
    }
  } else {
    for (int64_t i = i0; i < x.n; ++i) {
      float p = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x.p)[i]) : static_cast<const float*>(x.p)[i];
      float m = x.m[i], v = x.v[i];
      adamw_one(p, x.g[i], m, v, c);
      x.m[i] = m;
      x.v[i] = v;
      if constexpr (BF16)
        static_cast<uint16_t*>(x.p)[i] = (uint16_t)(pack_bf16x2(p, 0.0f) & 0xffffu);
      else
        static_cast<float*>(x.p)[i] = p;
    }
  }
}

}  // namespace

uint32_t adamw_blocks(int64_t n) {
  const int64_t per = (int64_t)kAdamwThreads * kAdamwPerThread;
  return (uint32_t)((n + per - 1) / per);
}

hipError_t launch_adamw(AdamwArgs a, bool param_bf16, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int64_t step, hipStream_t st) {
  // the step constants, one binary32 rounding each (the bias-correction
  // powers are evaluated in fp64)
  Step c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.eps = eps;
  const float lw = lr * weight_decay;
  c.decay = 1.0f - lw;
  c.omb1 = 1.0f - beta1;
  c.omb2 = 1.0f - beta2;
  const float bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  const float bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  c.sbc2 = std::sqrt(bc2);
  c.step_size = lr / bc1;
  uint32_t total = 0;
  for (int i = 0; i < a.count; ++i) {
    a.block0[i] = total;
    total += adamw_blocks(a.t[i].n);
  }
  for (int i = a.count; i <= kAdamwMaxTensors; ++i) a.block0[i] = total;
  if (total == 0) return hipSuccess;
  return param_bf16 ? timed_launch(kKernAdamw, adamw_kernel<true>, dim3(total), dim3(kAdamwThreads), st, a, c)
                    : timed_launch(kKernAdamw, adamw_kernel<false>, dim3(total), dim3(kAdamwThreads), st, a, c);
}

}  // namespace qnf4
