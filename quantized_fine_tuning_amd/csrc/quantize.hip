// NF4 blockwise quantization, double quantization of the block constants and
// standalone dequantization, for gfx950.
//
// Quantization (P4 §三 English derivation): per block of 64 consecutive
// elements c = max|w|, x = w / c, code = the nearest of 16 levels (ties to the
// lower index; a zero block gets the zero level).  Double quantization (P4 §二
// and §三): the fp32 block constants are re-quantized to an 8-bit float with a
// second-level block of 256 — here OCP E4M3 of the mean-centred constants with
// one fp32 scale per 256 and one fp32 mean per tensor.
//
// Kernels
//   nf4_quantize_kernel   one workgroup per 256 consecutive blocks (the DQ
//                         group size, a power of two); 16-byte coalesced loads,
//                         16 (fp32 input) or 8 (bf16 input) lanes per block,
//                         absmax by xor shuffles; writes packed codes, the fp32
//                         absmax (workspace) and the chunk's fp64 pairwise sum.
//   tree_level_kernel     fp64 pairwise sums of aligned groups of 1024 values,
//                         only while more than 16 groups of them remain.
//   dq_encode_kernel      every workgroup sums the remaining partial sums
//                         itself in the same tree order and takes
//                         mu = fl32(S / nb); then one wave per 256
//                         constants: d = c - mu, group max, s = max / 448,
//                         e = E4M3(d / s).
//   nf4_dequant_kernel    32 elements per thread, 16-byte loads of codes,
//                         64-byte contiguous stores of bf16.
#include <algorithm>
#include <type_traits>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int kChunkBlocks = 256;  // blocks per quantize workgroup
constexpr int kLevelGroup = 1024;  // values per tree_level workgroup
constexpr int kTailGroups = 16;    // groups the encode kernel sums itself

template <typename WT>
struct QTraits;
template <>
struct QTraits<float> {
  static constexpr int kEpl = 4;  // elements per lane (16 bytes)
  __device__ static float to_f32(float v) { return v; }
};
template <>
struct QTraits<uint16_t> {
  static constexpr int kEpl = 8;
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
};

// Codes through a table.  code(x) = #{j : x > t_j} for the sorted fp32
// thresholds t_0 < ... < t_14; every |t_j| > 2^-5, so |x| < 2^-5 has the zero
// code 7.  For 2^-5 <= |x| <= 1, cut each binade [2^e, 2^(e+1)) of |x| into
// 8 cells by the top 3 mantissa bits (bits 20..30 of |x| index the cell):
// 41 cells per sign, and no cell holds more than one threshold (codebook()
// checks this when it builds the thresholds and stops the process if not).  Cell c of a sign stores base = the count of
// thresholds below the whole cell and t* = the threshold inside it (or +inf):
// code(x) = base + (x > t*).  Cell 0 of each sign covers |x| < 2^-5 (base
// 7, t* = +inf).  Table: 42 cells for x >= 0, then 42 for x < 0.
constexpr int kCodeCells = 42;
constexpr int kCellBias = (122 << 3) - 1;  // bits 20..30 of 2^-5, minus one
__device__ __forceinline__ uint2 code_cell(int c, const Codebook& cb) {
  const int neg = c / kCodeCells, i = c % kCodeCells;
  if (i == 0) return make_uint2(0x7f800000u, 7u);
  const float lo = __uint_as_float((uint32_t)(kCellBias + i) << 20);
  const float hi = __uint_as_float((uint32_t)(kCellBias + i + 1) << 20);
  uint32_t base = 0;
  float tstar = __int_as_float(0x7f800000);  // +inf
  for (int j = 0; j < 15; ++j) {
    const float t = cb.t[j];
    if (!neg) {  // cell [lo, hi)
      if (t < lo) ++base;
      else if (t < hi) tstar = t;
    } else {  // cell (-hi, -lo]
      if (t <= -hi) ++base;
      else if (t <= -lo) tstar = t;
    }
  }
  return make_uint2(__float_as_uint(tstar), base);
}
// table index of x (no branch: |x| < 2^-5 clamps to cell 0)
__device__ __forceinline__ int code_cell_index(float x) {
  const uint32_t u = __float_as_uint(x);
  const int mag = max((int)((u & 0x7fffffffu) >> 20) - kCellBias, 0);
  return mag + (int)(u >> 31) * kCodeCells;
}

// max over the aligned group of LPB lanes (LPB = 8 or 16) of non-negative
// floats, as integers (same order), with DPP lane moves: xor 1 and 2 within
// quads, then mirrors within half rows and rows
template <int LPB>
__device__ __forceinline__ float group_max(float m) {
  uint32_t v = __float_as_uint(m);
  auto mv = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, decltype(ctrl)::value, 0xf, 0xf, false);
  };
  v = max(v, mv(v, std::integral_constant<int, 0xB1>()));   // quad_perm [1,0,3,2]
  v = max(v, mv(v, std::integral_constant<int, 0x4E>()));   // quad_perm [2,3,0,1]
  v = max(v, mv(v, std::integral_constant<int, 0x141>()));  // row_half_mirror
  if constexpr (LPB == 16) v = max(v, mv(v, std::integral_constant<int, 0x140>()));  // row_mirror
  return __uint_as_float(v);
}

template <typename WT>
__global__ __launch_bounds__(256) void nf4_quantize_kernel(const WT* __restrict__ W, int64_t nb,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax,
                                                           double* __restrict__ partial,
                                                           Codebook cb) {
  constexpr int EPL = QTraits<WT>::kEpl;
  constexpr int LPB = kBlock / EPL;      // lanes per block
  constexpr int BPW = 64 / LPB;          // blocks per wave per iteration
  constexpr int BPI = 4 * BPW;           // blocks per workgroup per iteration
  constexpr int ITERS = kChunkBlocks / BPI;
  static_assert(LPB == 8 || LPB == 16, "lanes per block");

  __shared__ float s_c[kChunkBlocks];
  __shared__ double s_w[4];
  __shared__ uint2 s_tab[2 * kCodeCells];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = lane % LPB, bl = lane / LPB;
  const int64_t chunk0 = (int64_t)blockIdx.x * kChunkBlocks;

  // a ring of RING loads in flight per lane (buffer loads: blocks past the
  // tensor read as zeros): few registers, so that many workgroups fit on a
  // compute unit and the grid runs in few rounds
  constexpr int RING = 3;
  const rsrc_t rw = make_rsrc(W + chunk0 * kBlock, (nb - chunk0) * kBlock * (int64_t)sizeof(WT));
  const uint32_t voff = (uint32_t)(((wave * BPW + bl) * kBlock + sub * EPL) * sizeof(WT));
  u32x4_t raw[RING];
#pragma unroll
  for (int it = 0; it < RING; ++it) raw[it] = buf_load16(rw, voff, (uint32_t)(it * BPI * kBlock * sizeof(WT)));
  if (tid < 2 * kCodeCells) s_tab[tid] = code_cell(tid, cb);
  __syncthreads();

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int local = it * BPI + wave * BPW + bl;
    const int64_t b = chunk0 + local;
    WT v[EPL];
    __builtin_memcpy(v, &raw[it % RING], sizeof(v));
    if (it + RING < ITERS)
      raw[it % RING] = buf_load16(rw, voff, (uint32_t)((it + RING) * BPI * kBlock * sizeof(WT)));
    float w[EPL];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      w[i] = QTraits<WT>::to_f32(v[i]);
      m = fmaxf(m, fabsf(w[i]));
    }
    m = group_max<LPB>(m);

    // x = fl32(w / m), the correctly rounded quotient, from one correctly
    // rounded reciprocal per block: q = w·y, then two residual corrections
    // r = w - q·m (exact with an FMA), q = q + r·y.  After the first, q is
    // within an ulp of w/m; with y = fl32(1/m) the second then gives the
    // correctly rounded quotient (Markstein's theorem).  A block with a tiny
    // absmax is scaled by 2^64 first (exact) so that y stays finite, and an
    // all-zero block divides by 1 (every x is 0: the zero code).
    const float sc = m < 0x1p-100f ? 0x1p64f : 1.0f;
    const float den = m != 0.0f ? m * sc : 1.0f;
    const float y = 1.0f / den;
    float x[EPL];
    uint2 cell[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float ws = w[i] * sc;
      float q = ws * y;
      q = __builtin_fmaf(__builtin_fmaf(-q, den, ws), y, q);
      x[i] = __builtin_fmaf(__builtin_fmaf(-q, den, ws), y, q);
      cell[i] = s_tab[code_cell_index(x[i])];
    }
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      packed |= (cell[i].y + (x[i] > __uint_as_float(cell[i].x) ? 1u : 0u)) << (4 * i);
    if (b < nb) {
      uint8_t* dst = codes + b * (kBlock / 2) + sub * (EPL / 2);
      if constexpr (EPL == 4) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = packed;
      }
      if (sub == 0) absmax[b] = m;
    }
  if (sub == 0) s_c[local] = (b < nb) ? m : 0.0f;
  }
  __syncthreads();

  // fp64 balanced pairwise sum of the chunk's 256 constants (block order)
  double v = (double)s_c[tid];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  if (tid == 0) partial[blockIdx.x] = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

// Pairwise fp64 sum of aligned group g of 1024 inputs (zero beyond n_in), by
// a workgroup of 256 threads: every thread returns the same S.
__device__ __forceinline__ double group_sum(const double* in, int64_t n_in, int64_t g, double* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = g * kLevelGroup + 4 * tid;
  double x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (base + i < n_in) ? in[base + i] : 0.0;
  double v = (x[0] + x[1]) + (x[2] + x[3]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  const double S = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
  __syncthreads();  // s_w is reused by the next call
  return S;
}

// One level of the tree: pairwise fp64 sums of aligned groups of 1024 inputs.
__global__ __launch_bounds__(256) void tree_level_kernel(const double* __restrict__ in, int64_t n_in,
                                                         double* __restrict__ out) {
  __shared__ double s_w[4];
  const double S = group_sum(in, n_in, blockIdx.x, s_w);
  if (threadIdx.x == 0) out[blockIdx.x] = S;
}

// The last levels of the tree, then the encode.  Every workgroup sums the
// n_in (<= kLevelGroup * kTailGroups) remaining partial sums itself, level by
// level in the same pairwise order as tree_level_kernel (the same S in every
// workgroup), and takes mu = fl32(S / nb); workgroup 0 also stores mu.  Then
// one wave per 256-constant group: d = c - mu, group max, s = max / 448,
// e = E4M3(d / s).
__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ absmax, int64_t nb,
                                                        const double* __restrict__ part, int64_t n_in,
                                                        float* __restrict__ mu_out,
                                                        uint8_t* __restrict__ e,
                                                        float* __restrict__ s_out, int64_t ng) {
  __shared__ double s_w[4];
  __shared__ double s_lv[kTailGroups];
  const int lane = threadIdx.x & 63;
  double S;
  {
    const int64_t n1 = (n_in + kLevelGroup - 1) / kLevelGroup;
    for (int64_t gi = 0; gi < n1; ++gi) {
      const double v = group_sum(part, n_in, gi, s_w);
      if (threadIdx.x == 0) s_lv[gi] = v;
    }
    __syncthreads();
    S = n1 == 1 ? s_lv[0] : group_sum(s_lv, n1, 0, s_w);
  }
  const float mu = (float)(S / (double)nb);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ng) return;
  const int64_t i0 = g * kDqBlock + 4 * lane;
  float d[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[i] = (i0 + i < nb) ? __fsub_rn(absmax[i0 + i], mu) : 0.0f;
    m = fmaxf(m, fabsf(d[i]));
  }
  m = wave_max(m);
  const float s = m / 448.0f;
  uint32_t word = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= f32_to_e4m3(d[i] / s) << (8 * i);
  }
  if (i0 + 4 <= nb) {
    *reinterpret_cast<uint32_t*>(e + i0) = word;
  } else {
    for (int i = 0; i < 4; ++i)
      if (i0 + i < nb) e[i0 + i] = (uint8_t)(word >> (8 * i));
  }
  if (lane == 0) s_out[g] = s;
}

// 32 elements (16 bytes of codes, half a block) per thread.
// Comparison formats (one fp32 absmax per 64-block, no double
// quantization): FMT 1 = NF4 codes (the codes of nf4_quantize_kernel), 2 =
// absmax INT4 (k = round(fl32(w · fl32(7/c))), halves away from zero, nibble
// k + 8), 3 = absmax INT8 (the same with 127, one byte per weight).  One
// group of LPB lanes per block and iteration, grid-stride over the blocks.
// (from the exact fraction p - trunc(p): floor(|p| + 0.5) would round the
// sum itself, e.g. 0.5 - 2^-25 + 0.5 ties to 1.0 in binary32)
__device__ __forceinline__ int round_half_away(float p) {
  const float t = __builtin_truncf(p);
  const int k = (int)t;
  const float d = __fsub_rn(p, t);  // exact
  return d >= 0.5f ? k + 1 : (d <= -0.5f ? k - 1 : k);
}

template <typename WT, int FMT>
__global__ __launch_bounds__(256) void format_quantize_kernel(const WT* __restrict__ W, int64_t nb,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ absmax, Codebook cb) {
  constexpr int EPL = QTraits<WT>::kEpl;
  constexpr int LPB = kBlock / EPL;
  __shared__ uint2 s_tab[2 * kCodeCells];
  if (FMT == 1 && threadIdx.x < 2 * kCodeCells) s_tab[threadIdx.x] = code_cell(threadIdx.x, cb);
  __syncthreads();
  const int sub = threadIdx.x % LPB;
  const int64_t groups = (int64_t)gridDim.x * (256 / LPB);
  for (int64_t b = (int64_t)blockIdx.x * (256 / LPB) + threadIdx.x / LPB; b - (threadIdx.x / LPB) < nb;
       b += groups) {
    // (the loop bound keeps the whole wave in the loop while any of its
    // blocks is in range, so that the max over lanes sees complete groups)
    const bool live = b < nb;
    WT v[EPL];
    if (live) {
      __builtin_memcpy(v, W + b * kBlock + sub * EPL, sizeof(v));
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i] = WT(0);
    }
    float w[EPL];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      w[i] = QTraits<WT>::to_f32(v[i]);
      m = fmaxf(m, fabsf(w[i]));
    }
    m = group_max<LPB>(m);
    uint32_t code[EPL];
    if constexpr (FMT == 1) {
      // x = fl32(w / m), then the nearest level through the cell table
      const float den = m != 0.0f ? m : 1.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float x = __fdiv_rn(w[i], den);
        const uint2 cell = s_tab[code_cell_index(x)];
        code[i] = cell.y + (x > __uint_as_float(cell.x) ? 1u : 0u);
      }
    } else {
      constexpr float qmax = FMT == 2 ? 7.0f : 127.0f;
      const float alpha = m != 0.0f ? __fdiv_rn(qmax, m) : 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int k = min(max(round_half_away(__fmul_rn(w[i], alpha)), -(int)qmax), (int)qmax);
        code[i] = FMT == 2 ? (uint32_t)(k + 8) : (uint32_t)k & 0xffu;
      }
    }
    if (!live) continue;
    if constexpr (FMT == 3) {
      uint8_t* dst = codes + b * kBlock + sub * EPL;
      if constexpr (EPL == 4) {
        *reinterpret_cast<uint32_t*>(dst) = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      } else {
        *reinterpret_cast<u32x2_t*>(dst) =
            u32x2_t{code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                    code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24)};
      }
    } else {
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) packed |= code[i] << (4 * i);
      uint8_t* dst = codes + b * (kBlock / 2) + sub * (EPL / 2);
      if constexpr (EPL == 4) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = packed;
      }
    }
    if (sub == 0) absmax[b] = m;
  }
}

template <bool F16>
__global__ __launch_bounds__(256) void nf4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ e,
                                                          const float* __restrict__ s,
                                                          const float* __restrict__ mu_p,
                                                          int64_t n_units, uint16_t* __restrict__ out,
                                                          Codebook cb) {
  __shared__ float s_q[16];
  if (threadIdx.x < 16) s_q[threadIdx.x] = cb.q[threadIdx.x];
  __syncthreads();
  const float mu = *mu_p;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(codes + u * 16);
    const int64_t b = u >> 1;  // 2 units per 64-block
    const float cp = decode_constant(e[b], s[b / kDqBlock], mu);
    u32x4_t o[4];
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      uint32_t r[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = __fmul_rn(s_q[(w[wi] >> (8 * p)) & 15u], cp);
        const float c = __fmul_rn(s_q[(w[wi] >> (8 * p + 4)) & 15u], cp);
        r[p] = pack16<F16>(a, c);
      }
      o[wi] = u32x4_t{r[0], r[1], r[2], r[3]};
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + u * 32);
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) dst[wi] = o[wi];
  }
}

}  // namespace

QuantLayout quant_layout(int64_t N, int64_t K) {
  QuantLayout L{};
  L.nb = N * K / kBlock;
  L.ng = (L.nb + kDqBlock - 1) / kDqBlock;
  L.chunks = (L.nb + kChunkBlocks - 1) / kChunkBlocks;
  int64_t n = L.chunks;
  int i = 0;
  do {
    n = (n + kLevelGroup - 1) / kLevelGroup;
    L.lvl_len[i++] = n;
  } while (n > 1 && i < 7);
  L.lvl_len[i] = 0;
  size_t off = 0;
  L.off_absmax = off;
  off += round_up(L.chunks * kChunkBlocks * 4, 256);
  L.off_partial = off;
  off += round_up(L.chunks * 8, 256);
  L.off_lvl_a = off;
  off += round_up(L.lvl_len[0] * 8, 256);
  L.off_lvl_b = off;
  off += round_up(L.lvl_len[0] * 8, 256);
  L.total = off;
  return L;
}

hipError_t launch_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* e, float* s, float* mu, char* ws, const QuantLayout& L,
                           hipStream_t st) {
  float* absmax = reinterpret_cast<float*>(ws + L.off_absmax);
  double* partial = reinterpret_cast<double*>(ws + L.off_partial);
  double* lvl[2] = {reinterpret_cast<double*>(ws + L.off_lvl_a),
                    reinterpret_cast<double*>(ws + L.off_lvl_b)};
  const Codebook& cb = codebook();
  {
    hipError_t e = w_bf16 ? timed_launch(kKernQuantize, nf4_quantize_kernel<uint16_t>, dim3((unsigned)L.chunks),
                                         dim3(256), st, static_cast<const uint16_t*>(W), L.nb, codes,
                                         absmax, partial, cb)
                          : timed_launch(kKernQuantize, nf4_quantize_kernel<float>, dim3((unsigned)L.chunks),
                                         dim3(256), st, static_cast<const float*>(W), L.nb, codes, absmax,
                                         partial, cb);
    if (e != hipSuccess) return e;
  }
  // tree levels of their own only while more partial sums remain than the
  // encode kernel sums itself
  const double* in = partial;
  int64_t n_in = L.chunks;
  for (int i = 0; n_in > (int64_t)kLevelGroup * kTailGroups; ++i) {
    const int64_t n_out = (n_in + kLevelGroup - 1) / kLevelGroup;
    double* out = lvl[i & 1];
    tree_level_kernel<<<(unsigned)n_out, 256, 0, st>>>(in, n_in, out);
    in = out;
    n_in = n_out;
  }
  dq_encode_kernel<<<(unsigned)((L.ng + 3) / 4), 256, 0, st>>>(absmax, L.nb, in, n_in, mu, e, s, L.ng);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* e, const float* s,
                             const float* mu, int64_t N, int64_t K, uint16_t* out, bool f16,
                             hipStream_t st) {
  const int64_t units = N * K / 32;
  int64_t grid = (units + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (f16)
    nf4_dequant_kernel<true><<<(unsigned)grid, 256, 0, st>>>(codes, e, s, mu, units, out, codebook());
  else
    nf4_dequant_kernel<false><<<(unsigned)grid, 256, 0, st>>>(codes, e, s, mu, units, out, codebook());
  return hipGetLastError();
}

hipError_t launch_format_quantize(const void* W, bool w_bf16, int64_t N, int64_t K, int fmt, uint8_t* codes,
                                  float* absmax, hipStream_t st) {
  const int64_t nb = N * K / kBlock;
  if (nb == 0) return hipSuccess;
  const int per_wg = w_bf16 ? 256 / (kBlock / 8) : 256 / (kBlock / 4);  // blocks per workgroup and pass
  const unsigned grid = (unsigned)std::min<int64_t>((nb + per_wg - 1) / per_wg, 256 * 16);
  const Codebook& cb = codebook();
#define QNF4_FQ(WT, F) format_quantize_kernel<WT, F><<<grid, 256, 0, st>>>(static_cast<const WT*>(W), nb, codes, absmax, cb)
  if (w_bf16) {
    if (fmt == 1) QNF4_FQ(uint16_t, 1); else if (fmt == 2) QNF4_FQ(uint16_t, 2); else QNF4_FQ(uint16_t, 3);
  } else {
    if (fmt == 1) QNF4_FQ(float, 1); else if (fmt == 2) QNF4_FQ(float, 2); else QNF4_FQ(float, 3);
  }
#undef QNF4_FQ
  return hipGetLastError();
}

}  // namespace qnf4
