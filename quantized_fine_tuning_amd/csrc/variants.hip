// Comparison formats of the frozen weight, gfx950: dequantization and the
// dequant-GEMV for few tokens.
//
// P2 §4.1 and P4 (trade-off ②): NF4 against ordinary uniform 4-bit integer
// quantization; P3 (公式导读 2): absmax INT8; P4 §三: NF4's per-block fp32
// constants before double quantization.  All three formats keep one fp32
// absmax c per 64-block; a weight is w' = RNE_bf16(fl32(L[code]·c)) with
//   FMT 1 (NF4, double quantization off): L = the 16 NF4 levels;
//   FMT 2 (absmax INT4): code k + 8, L = fl32(k / 7), k in [-7, 7];
//   FMT 3 (absmax INT8): one byte k (two's complement), L = fl32(k / 127).
//
//   format_dequant_kernel  32 weights per thread: 16- or 32-byte loads of
//                          codes, 64-byte stores of bf16.
//   format_gemv_kernel     Y = X·Ŵᵀ for M <= 16 tokens, the layout of the NF4
//                          GEMV: one workgroup of 16 waves per 16 weight rows;
//                          lane (row l % 16, q = l / 16) owns whole blocks (64
//                          codes and their constant); a group of 4 blocks of
//                          the 16 rows feeds 8 v_mfma_f32_16x16x32_bf16 whose A
//                          operand is X padded to 16 rows; the 16 partial
//                          tiles are summed in a fixed order.  Levels come from
//                          an LDS table (16 or 256 fp32 values).
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int kFmtNf4 = 1, kFmtInt4 = 2, kFmtInt8 = 3;

template <int FMT>
struct Fmt {
  static constexpr int kLevels = FMT == kFmtInt8 ? 256 : 16;
  static constexpr int kBlockBytes = FMT == kFmtInt8 ? 64 : 32;  // code bytes per 64-block
};

// the level table: NF4 levels, or k / qmax for the integer formats
template <int FMT>
__device__ __forceinline__ float level(int i, const Codebook& cb) {
  if constexpr (FMT == kFmtNf4) {
    return cb.q[i];
  } else if constexpr (FMT == kFmtInt4) {
    const int k = i - 8;
    return k >= -7 ? __fdiv_rn((float)k, 7.0f) : 0.0f;
  } else {
    const int k = (int)(int8_t)(uint8_t)i;
    return k >= -127 ? __fdiv_rn((float)k, 127.0f) : 0.0f;
  }
}

// the code of weight e of a 32-bit word of codes (8 nibbles or 4 bytes)
template <int FMT>
__device__ __forceinline__ uint32_t code_of(uint32_t w, int e) {
  if constexpr (FMT == kFmtInt8) {
    return (w >> (8 * e)) & 0xffu;
  } else {
    return (w >> (4 * e)) & 15u;
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void format_dequant_kernel(const uint8_t* __restrict__ codes,
                                                             const float* __restrict__ absmax, int64_t n_units,
                                                             uint16_t* __restrict__ out, Codebook cb) {
  constexpr int WPW = FMT == kFmtInt8 ? 4 : 8;  // weights per 32-bit word of codes
  __shared__ float s_l[Fmt<FMT>::kLevels];
  for (int i = threadIdx.x; i < Fmt<FMT>::kLevels; i += blockDim.x) s_l[i] = level<FMT>(i, cb);
  __syncthreads();
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    // unit u: weights 32u .. 32u + 31 (half a block)
    const float c = absmax[u >> 1];
    constexpr int UB = FMT == kFmtInt8 ? 32 : 16;  // code bytes per unit
    uint32_t w[32 / WPW];
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(codes + u * UB);
#pragma unroll
    for (int i = 0; i < 32 / WPW / 4; ++i) {
      const u32x4_t v = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[4 * i + j] = v[j];
    }
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int e0 = 2 * p, e1 = 2 * p + 1;
      const float a = __fmul_rn(s_l[code_of<FMT>(w[e0 / WPW], e0 % WPW)], c);
      const float b = __fmul_rn(s_l[code_of<FMT>(w[e1 / WPW], e1 % WPW)], c);
      o[p] = pack_bf16x2(a, b);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + u * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4_t{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
}

constexpr int kFgWaves = 16, kFgThreads = 64 * kFgWaves, kFgRows = 16;

template <int FMT>
__global__ __launch_bounds__(kFgThreads) void format_gemv_kernel(const uint8_t* __restrict__ codes,
                                                                 const float* __restrict__ absmax, int64_t N,
                                                                 int64_t K, const uint16_t* __restrict__ X, int M,
                                                                 void* __restrict__ Y, int y_bf16, Codebook cb) {
  constexpr int BB = Fmt<FMT>::kBlockBytes, NV = BB / 16;  // 16-byte loads per block
  __shared__ float s_l[Fmt<FMT>::kLevels];
  __shared__ f32x4_t s_acc[kFgWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kFgRows;
  const int64_t nb = K / kBlock;         // blocks per row
  const int64_t ngroups = (nb + 3) / 4;  // groups of 4 blocks per row
  // rows past N read as zero
  const rsrc_t rc = make_rsrc(codes + n0 * nb * BB, (N - n0) * nb * BB);
  const rsrc_t ra = make_rsrc(absmax + n0 * nb, (N - n0) * nb * 4);
  const rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const bool x_row = lr < M;

  struct Group {
    u32x4_t c[NV];  // the lane's 64 codes
    float a;        // its absmax
    u32x4_t x[8];   // X fragments of the 8 MFMAs (zero if lr >= M)
  };
  auto load = [&](Group& g, int64_t grp) __attribute__((always_inline)) {
    const int64_t b = 4 * grp + kq;  // this lane's block in its row
    const bool ok = grp < ngroups && b < nb;
    const uint32_t co = ok ? (uint32_t)((lr * nb + b) * BB) : 0x7fffffffu;
#pragma unroll
    for (int i = 0; i < NV; ++i) g.c[i] = buf_load16(rc, co, 16u * i);
    g.a = __uint_as_float(buf_load4(ra, ok ? (uint32_t)((lr * nb + b) * 4) : 0x7fffffffu, 0u));
#pragma unroll
    for (int t = 0; t < 8; ++t) g.x[t] = u32x4_t{0u, 0u, 0u, 0u};
    if (x_row) {
      const uint32_t xo = ok ? (uint32_t)((lr * K + b * kBlock) * 2) : 0x7fffffffu;
#pragma unroll
      for (int t = 0; t < 8; ++t) g.x[t] = buf_load16(rx, xo, 16u * t);
    }
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Group& g) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // codes 8t .. 8t + 7 of the lane's block: one word of nibbles, or two
      // words of bytes
      uint32_t w[2];
      if constexpr (FMT == kFmtInt8) {
        w[0] = g.c[t >> 1][2 * (t & 1)];
        w[1] = g.c[t >> 1][2 * (t & 1) + 1];
      } else {
        w[0] = g.c[t >> 2][t & 3];
      }
      u32x4_t bfrag;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 2 * p, e1 = 2 * p + 1;
        uint32_t c0, c1;
        if constexpr (FMT == kFmtInt8) {
          c0 = code_of<FMT>(w[e0 >> 2], e0 & 3);
          c1 = code_of<FMT>(w[e1 >> 2], e1 & 3);
        } else {
          c0 = code_of<FMT>(w[0], e0);
          c1 = code_of<FMT>(w[0], e1);
        }
        bfrag[p] = pack_bf16x2(__fmul_rn(s_l[c0], g.a), __fmul_rn(s_l[c1], g.a));
      }
      acc = mfma_16x16x32(g.x[t], bfrag, acc);
    }
  };

  Group ga, gb;
  load(ga, wave);
  for (int i = tid; i < Fmt<FMT>::kLevels; i += kFgThreads) s_l[i] = level<FMT>(i, cb);
  __syncthreads();  // level table
  // two groups per iteration, alternating buffers: the next group's loads are
  // issued before the current one is consumed
  for (int64_t grp = wave; grp < ngroups; grp += 2 * kFgWaves) {
    load(gb, grp + kFgWaves);
    __builtin_amdgcn_sched_barrier(0);
    consume(ga);
    if (grp + kFgWaves >= ngroups) break;
    load(ga, grp + 2 * kFgWaves);
    __builtin_amdgcn_sched_barrier(0);
    consume(gb);
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  // one thread per output (token m, weight row n0 + c): the 16 partial tiles
  // in a fixed order
  if (tid < 16 * kFgRows) {
    const int m = tid >> 4, c = tid & 15;
    const int64_t nn = n0 + c;
    if (m < M && nn < N) {
      float y = s_acc[0][16 * (m >> 2) + c][m & 3];
#pragma unroll
      for (int w = 1; w < kFgWaves; ++w) y = __fadd_rn(y, s_acc[w][16 * (m >> 2) + c][m & 3]);
      if (y_bf16)
        static_cast<uint16_t*>(Y)[(int64_t)m * N + nn] = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
      else
        static_cast<float*>(Y)[(int64_t)m * N + nn] = y;
    }
  }
}

}  // namespace

hipError_t launch_format_dequantize(const uint8_t* codes, const float* absmax, int fmt, int64_t N, int64_t K,
                                    uint16_t* out, hipStream_t st) {
  const int64_t units = N * K / 32;
  if (units == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((units + 255) / 256, 256 * 16);
  const Codebook& cb = codebook();
  if (fmt == kFmtNf4)
    format_dequant_kernel<kFmtNf4><<<grid, 256, 0, st>>>(codes, absmax, units, out, cb);
  else if (fmt == kFmtInt4)
    format_dequant_kernel<kFmtInt4><<<grid, 256, 0, st>>>(codes, absmax, units, out, cb);
  else
    format_dequant_kernel<kFmtInt8><<<grid, 256, 0, st>>>(codes, absmax, units, out, cb);
  return hipGetLastError();
}

hipError_t launch_format_gemv(const uint8_t* codes, const float* absmax, int fmt, int64_t N, int64_t K,
                              const uint16_t* X, int64_t M, void* Y, bool y_bf16, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)((N + kFgRows - 1) / kFgRows));
  const Codebook& cb = codebook();
  if (fmt == kFmtNf4)
    return timed_launch(kKernFormatGemv, format_gemv_kernel<kFmtNf4>, grid, dim3(kFgThreads), st, codes, absmax, N,
                        K, X, (int)M, Y, y_bf16 ? 1 : 0, cb);
  if (fmt == kFmtInt4)
    return timed_launch(kKernFormatGemv, format_gemv_kernel<kFmtInt4>, grid, dim3(kFgThreads), st, codes, absmax,
                        N, K, X, (int)M, Y, y_bf16 ? 1 : 0, cb);
  return timed_launch(kKernFormatGemv, format_gemv_kernel<kFmtInt8>, grid, dim3(kFgThreads), st, codes, absmax, N,
                      K, X, (int)M, Y, y_bf16 ? 1 : 0, cb);
}

}  // namespace qnf4
