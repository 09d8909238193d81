// Sum of the split-reduction partials of the dequant-in-tile GEMMs (few
// tokens, see tiling.h): out[i] = P[0][i] + P[1][i] + ... + P[S-1][i], added in
// split order in fp32 (the same result on every run), then stored as fp32 or
// rounded once to the 16-bit compute format.  Streaming, four outputs per
// lane and access.
#include "host.h"

namespace qnf4 {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kReduceMaxBlocks = 2048;

template <bool F16>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const f32x4_t* __restrict__ P, int splits,
                                                                       int64_t n4, void* __restrict__ out,
                                                                       int out16) {
  const int64_t stride = (int64_t)gridDim.x * kReduceThreads;
  for (int64_t i = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x; i < n4; i += stride) {
    f32x4_t a = __builtin_nontemporal_load(P + i);
    // the loads of four partials are issued before their adds
    for (int s = 1; s < splits; s += 4) {
      f32x4_t b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // an existing partial whatever q, so that the loads are unconditional
        const int sq = s + q < splits ? s + q : splits - 1;
        b[q] = __builtin_nontemporal_load(P + (int64_t)sq * n4 + i);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (s + q < splits) {
          a[0] = a[0] + b[q][0];
          a[1] = a[1] + b[q][1];
          a[2] = a[2] + b[q][2];
          a[3] = a[3] + b[q][3];
        }
    }
    if (out16) {
      u32x2_t o;
      o[0] = pack16<F16>(a[0], a[1]);
      o[1] = pack16<F16>(a[2], a[3]);
      static_cast<u32x2_t*>(out)[i] = o;
    } else {
      static_cast<f32x4_t*>(out)[i] = a;
    }
  }
}

}  // namespace

// P holds `splits` partial arrays of n floats each (n % 4 == 0), back to back.
hipError_t launch_splitk_reduce(const float* P, int splits, int64_t n, void* out, bool out16, bool f16,
                                hipStream_t st) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  const int64_t want = (n4 + kReduceThreads - 1) / kReduceThreads;
  const unsigned blocks = (unsigned)(want < kReduceMaxBlocks ? want : kReduceMaxBlocks);
  const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(P);
  const int o16 = out16 ? 1 : 0;
  if (f16)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(blocks), dim3(kReduceThreads), 0, st, p4, splits, n4, out, o16);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(blocks), dim3(kReduceThreads), 0, st, p4, splits, n4, out,
                       o16);
  return hipGetLastError();
}

}  // namespace qnf4
