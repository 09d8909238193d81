// Dequant-GEMV forward for few tokens (M <= 16), gfx950.
//
// P2 §六 and P5 (follow-up 1): at inference the 4-bit weight is dequantized to
// 16 bit on the fly for every product; with few tokens the product is bound by
// streaming the packed codes from HBM, so this path reads each code exactly
// once and keeps everything else small.
//
//   lora_down_small_kernel  T[m][j] = Σ_k X[m][k]·A[j][k] in fp32, one
//                           workgroup per j, fixed-order reduction.
//   gemv_kernel             one workgroup per 16 weight rows, 4 waves splitting
//                           K round-robin by 64-blocks.  Each lane turns 16 codes
//                           (8 bytes) of one row into bf16 in registers and feeds
//                           them straight into v_mfma_f32_16x16x32_bf16 as the B
//                           operand (X rows padded to 16 are the A operand).  The
//                           four partial sums are combined in a fixed order and
//                           the LoRA term s·Σ_j T[m][j]·B[n][j] is added in fp32.
#include "host.h"

namespace qnf4 {
namespace {

__global__ __launch_bounds__(256) void lora_down_small_kernel(const uint16_t* __restrict__ X,
                                                              int M, int64_t K,
                                                              const uint16_t* __restrict__ A,
                                                              int r, float* __restrict__ T) {
  __shared__ float s_part[4][16];
  const int j = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * 256) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(A + (int64_t)j * K + k);
    float af[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[2 * i] = bf16lo(a[i]);
      af[2 * i + 1] = bf16hi(a[i]);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < M) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(X + (int64_t)m * K + k);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = __fadd_rn(s, __fmul_rn(bf16lo(x[i]), af[2 * i]));
          s = __fadd_rn(s, __fmul_rn(bf16hi(x[i]), af[2 * i + 1]));
        }
        acc[m] = __fadd_rn(acc[m], s);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __fadd_rn(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_part[wave][m] = v;
  }
  __syncthreads();
  if (tid < M) {
    const float v = __fadd_rn(__fadd_rn(s_part[0][tid], s_part[1][tid]),
                              __fadd_rn(s_part[2][tid], s_part[3][tid]));
    T[(int64_t)tid * r + j] = v;
  }
}

constexpr int GEMV_ROWS = 16;

__global__ __launch_bounds__(256) void gemv_kernel(Nf4View W, const uint16_t* __restrict__ X, int M,
                                                   const float* __restrict__ T,
                                                   const uint16_t* __restrict__ B, int r,
                                                   float scale, void* __restrict__ Y, int y_bf16,
                                                   Codebook cb) {
  __shared__ float sq[16];
  __shared__ f32x4_t s_acc[4][64];
  if (threadIdx.x < 16) sq[threadIdx.x] = cb.q[threadIdx.x];
  __syncthreads();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kq = lane >> 4;
  const int64_t K = W.K, N = W.N;
  const int64_t n = (int64_t)blockIdx.x * GEMV_ROWS + row;
  const bool row_ok = n < N;
  const int64_t nsteps = K / kBlock;
  const float mu = *W.mu;
  const uint8_t* crow = W.codes + (row_ok ? n : 0) * (K / 2);
  const uint16_t* xrow = X + (int64_t)(row < M ? row : 0) * K;
  const bool x_ok = row < M;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t st = wave; st < nsteps; st += 4) {
    u32x2_t cw = {0x77777777u, 0x77777777u};
    float cp = 0.0f;
    if (row_ok) {
      cw = *reinterpret_cast<const u32x2_t*>(crow + st * 32 + kq * 8);
      const int64_t b = n * nsteps + st;
      cp = decode_constant(W.e[b], W.s[b / kDqBlock], mu);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t w = cw[ks];
      u32x4_t bfrag;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = __fmul_rn(sq[(w >> (8 * p)) & 15u], cp);
        const float c = __fmul_rn(sq[(w >> (8 * p + 4)) & 15u], cp);
        bfrag[p] = pack_bf16x2(a, c);
      }
      u32x4_t afrag = {0u, 0u, 0u, 0u};
      if (x_ok) afrag = *reinterpret_cast<const u32x4_t*>(xrow + st * kBlock + kq * 16 + ks * 8);
      acc = mfma_16x16x32(afrag, bfrag, acc);
    }
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4_t a0 = s_acc[0][lane], a1 = s_acc[1][lane], a2 = s_acc[2][lane],
                  a3 = s_acc[3][lane];
    // lane holds D rows (tokens) 4*(lane/16)+v of column (weight row) lane%16
    const int64_t nn = (int64_t)blockIdx.x * GEMV_ROWS + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * (lane >> 4) + v;
      if (m < M && nn < N) {
        float y = __fadd_rn(__fadd_rn(a0[v], a1[v]), __fadd_rn(a2[v], a3[v]));
        float l = 0.0f;
        for (int j = 0; j < r; ++j)
          l = __fadd_rn(l, __fmul_rn(T[(int64_t)m * r + j], bf16_to_f32(B[nn * r + j])));
        y = __fadd_rn(y, __fmul_rn(scale, l));
        if (y_bf16)
          static_cast<uint16_t*>(Y)[(int64_t)m * N + nn] = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
        else
          static_cast<float*>(Y)[(int64_t)m * N + nn] = y;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float scale, void* Y, bool y_bf16, float* T,
                       hipStream_t st) {
  lora_down_small_kernel<<<(unsigned)r, 256, 0, st>>>(X, (int)M, W.K, A, r, T);
  const unsigned grid = (unsigned)((W.N + GEMV_ROWS - 1) / GEMV_ROWS);
  {
    TimedLaunch tl(kKernGemv, st);
    gemv_kernel<<<grid, 256, 0, st>>>(W, X, (int)M, T, B, r, scale, Y, y_bf16 ? 1 : 0, codebook());
  }
  return hipGetLastError();
}

}  // namespace qnf4
