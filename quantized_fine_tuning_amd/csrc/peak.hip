// Benchmark instrumentation: the two in-run reference points the roofline
// fractions are also reported against.
//
//   mfma_peak_kernel   v_mfma_f32_16x16x32_bf16 issued back to back from
//                      registers (8 independent accumulators per wave, so the
//                      matrix pipe never waits on a result), on every SIMD
//                      of every compute unit: the bf16 dense MFMA rate the
//                      chip sustains at the clock it runs at under that load.
//                      The first lane of workgroup 0 reads the shader clock
//                      counter and the constant-rate real-time counter before
//                      and after its loop, which gives that clock.
//   stream_copy_kernel a plain copy, 16 bytes per lane and access: the HBM
//                      rate of a streaming read + write of known size, also
//                      the calibration for the HBM byte counters.
#include "host.h"

namespace qnf4 {
namespace {

__global__ __launch_bounds__(256) void mfma_peak_kernel(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, w0 = 0;
  if (timer) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  u32x4_t a = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4_t b = {0x3c003c00u, 0x3c003c00u ^ (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  // distinct starting values: eight chains the compiler cannot merge (with
  // equal operands and equal starts it treats them as one value and
  // shuffles accumulator registers between the MFMAs)
  f32x4_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4_t{(float)(lane + 64 * i), 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma_16x16x32(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // never in practice: keeps the MFMAs
  if (timer) {
    asm volatile("" : "+v"(s));  // the loop's results exist before the clocks are read
    const uint64_t c1 = clock64(), w1 = wall_clock64();
    uint64_t* const clk = reinterpret_cast<uint64_t*>(sink + kPeakWorkgroups);
    clk[0] = c0;
    clk[1] = c1;
    clk[2] = w0;
    clk[3] = w1;
  }
}

// Four 16-byte loads in flight per lane before their stores.
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a0 = __builtin_nontemporal_load(src + i);
    const u32x4_t a1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t a2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t a3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a0, dst + i);
    __builtin_nontemporal_store(a1, dst + i + stride);
    __builtin_nontemporal_store(a2, dst + i + 2 * stride);
    __builtin_nontemporal_store(a3, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

int64_t mfma_peak_flop(int64_t iters) {
  return (int64_t)kPeakWorkgroups * 4 * iters * 8 * (16 * 16 * 32 * 2);
}

hipError_t launch_mfma_peak(int64_t iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kPeakWorkgroups), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(2048), dim3(256), 0, st, static_cast<const u32x4_t*>(src),
                     static_cast<u32x4_t*>(dst), n16);
  return hipGetLastError();
}

}  // namespace qnf4
