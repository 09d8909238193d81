// The LoRA adapter merged into the dequantized weight, gfx950.
//
// P5 (follow-up 1): for serving speed the fine-tuned model is converted once
// to 16 bits, the LoRA weights merged into the dequantized weight.  P1 §七
// (dataflow figure): the layer computes X·Ŵᵀ + s·(X·Aᵀ)·Bᵀ = X·(Ŵ + s·B·A)ᵀ.
// P1 §五: merging and re-quantizing can bring the quantization error back
// (re-quantization is the quantize entry point applied to the bf16 result).
//
//   W_m[n][k] = RND(fl32(ŵ[n][k] + fl32(s · Σ_j B[n][j]·A[j][k])))
//
// with ŵ = RNE_bf16(fl32(q[code]·c')) exactly as the forward pass multiplies
// it, the rank-r sum accumulated in fp32 by MFMA, and RND the round to nearest
// even into bf16 or fp16.  (Against the exact sum rounded once, the result is
// within one unit in the last place.)
//
// merge_kernel: one workgroup of 4 waves per tile of 64 rows x 256 columns.
//   * The rank-r product D[k][n] = Σ_j A[j][k]·B[n][j] runs in chunks of 64
//     ranks (two slices of 32), all of a chunk's loads issued before one
//     barrier: the A slices (32 x 256 each) copied from memory straight into
//     LDS, row-major, their MFMA fragments (8 consecutive ranks of one column)
//     gathered with 2-byte reads; the B slices (64 x 32) through registers
//     (two-byte loads: B's rows need not be aligned), whose rows are
//     fragments already.
//   * Wave w owns columns kw = k0 + 64w .. +63 (one NF4 block of each row)
//     against all 64 rows: 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  The
//     MFMA row i of column tile kf stands for column kw + 16(i / 4) + 4kf +
//     i % 4, so that lane (l % 16, q = l / 16), which receives MFMA rows
//     4q .. 4q+3 of every tile, ends with the 16 contiguous columns
//     kw + 16q .. +15 of its row: one 8-byte load of codes and two 16-byte
//     stores per row.
//   * The lane's codes, e4m3 constants and group scales are requested first,
//     so their latency overlaps the product.
#include "host.h"

namespace qnf4 {
namespace {

constexpr int kMergeRows = 64, kMergeCols = 256, kMergeThreads = 256;
constexpr int kMergeChunk = 64;  // ranks per chunk (two slices of 32)

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Byte offset of element (row, j) of a B slice (64-byte rows, 16-byte chunk c
// of row `row` at physical chunk c ^ ((row >> 1) & 3)): the 8 lanes of one
// 16-byte fragment read (rows 0..7 of a tile) hit distinct banks.
__device__ __forceinline__ uint32_t slice_off(int row, int j) {
  return (uint32_t)(row * 64 + (((j >> 3) ^ ((row >> 1) & 3)) << 4) + 2 * (j & 7));
}
// Byte offset of element (j, k) of an A slice (512-byte rows; in the rows of
// odd 8-row groups the 16-byte pieces swap in pairs, columns XOR 8): a
// gather of one rank by a quarter-wave reads 2 dwords in each of 4 banks
// groups 8 dwords apart, and the other quarter-wave of the half-wave (rows 8
// further) the 4 dwords beside them.
__device__ __forceinline__ uint32_t aslice_off(int j, int k) {
  return (uint32_t)(j * 512 + 2 * (k ^ (j & 8)));
}
// the column (within the wave's 64) that MFMA row i of column tile kf stands for
__device__ __forceinline__ int tile_col(int kf, int i) { return 16 * (i >> 2) + 4 * kf + (i & 3); }

template <bool F16>
__device__ __forceinline__ uint32_t pack_out(float a, float b) {
  if constexpr (F16) {
    f16x2_t h;
    h.x = (_Float16)a;  // v_cvt_f16_f32: nearest even, denormals kept
    h.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, h);
  } else {
    return pack_bf16x2(a, b);
  }
}

template <bool F16>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(Nf4View W, const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B, int r,
                                                              float scale, uint16_t* __restrict__ out,
                                                              uint32_t col_tiles, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) char s_a[2][32 * kMergeCols * 2];  // A slices [32 j][256 k]
  __shared__ __attribute__((aligned(16))) char s_b[2][kMergeRows * 64];       // B slices [64 n][32 j]
  __shared__ float s_q[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const int64_t N = W.N, K = W.K;
  const int64_t n0 = (int64_t)(blockIdx.x / col_tiles) * kMergeRows;
  const int64_t k0 = (int64_t)(blockIdx.x % col_tiles) * kMergeCols;
  const int64_t kw = k0 + 64 * wave;  // this wave's block column
  const bool k_in = kw < K;
  const int64_t kpr = K / kBlock;     // blocks per row

  // the lane's codes (columns kw + 16q .. +15: bytes 8q .. 8q+7 of the
  // block) and constants for its 4 rows; rows past N read zero, a wave past
  // K loads nothing
  const rsrc_t rc = make_rsrc(W.codes, N * K / 2);
  const rsrc_t re = make_rsrc(W.e, N * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  u32x2_t cw[4];
  uint32_t ee[4], ss[4];
#pragma unroll
  for (int nf = 0; nf < 4; ++nf) {
    const int64_t n = n0 + 16 * nf + lr;
    const int64_t b = n * kpr + kw / kBlock;
    const bool ok = k_in && n < N;
    cw[nf] = buf_load8(rc, ok ? (uint32_t)(b * (kBlock / 2) + 8 * q) : 0x7fffffffu, 0u);
    ee[nf] = buf_load1(re, ok ? (uint32_t)b : 0x7fffffffu, 0u);
    ss[nf] = buf_load4(rs, ok ? (uint32_t)((b / kDqBlock) * 4) : 0x7fffffffu, 0u);
  }
  if (tid < 16) s_q[tid] = cb.q[tid];

  const rsrc_t ra = make_rsrc(A, (int64_t)r * K * 2);
  const rsrc_t rb = make_rsrc(B, N * r * 2);
  // A copy: wave instruction c of slice h fills rows 2(4w + c) and +1 (1 KB);
  // lane i lands at byte 16i of them: row 2(4w + c) + i / 32, physical
  // piece i % 32, which holds logical columns 8((i % 32) ^ (row & 8 ? 1 : 0))
  const int crow0 = lane >> 5, cpiece = lane & 31;
  // B: thread t loads row t / 4, ranks 8(t % 4) .. +7 of each slice
  const int bnl = tid >> 2, bjc = 8 * (tid & 3);
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < r; c0 += kMergeChunk) {
    if (c0 > 0) __syncthreads();  // the previous chunk's reads are done
    uint32_t h[2][8];
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int j0 = c0 + 32 * hs;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int jj = 2 * (4 * wave + c) + crow0;
        const int kc = 8 * (cpiece ^ ((jj & 8) ? 1 : 0));
        const bool ok = j0 < r && j0 + jj < r && k0 + kc < K;
        buf_load_lds16(ra, s_a[hs] + 1024 * (4 * wave + c),
                       ok ? (uint32_t)(((int64_t)(j0 + jj) * K + k0 + kc) * 2) : 0x7fffffffu, 0u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + bjc + e;
        h[hs][e] = buf_load2(rb, j < r ? (uint32_t)(((n0 + bnl) * r + j) * 2) : 0x7fffffffu, 0u);
      }
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (h[hs][2 * e] & 0xffffu) | (h[hs][2 * e + 1] << 16);
      *reinterpret_cast<u32x4_t*>(s_b[hs] + slice_off(bnl, bjc)) = v;
    }
    wait_vmem();  // this wave's copies into LDS have landed
    __syncthreads();
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      if (c0 + 32 * hs >= r) break;
      // A fragment of column tile kf: MFMA row lr, ranks 8q .. +7
      u32x4_t a[4], bf[4];
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) {
        const int k = 64 * wave + tile_col(kf, lr);
        uint32_t g[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = *reinterpret_cast<const uint16_t*>(s_a[hs] + aslice_off(8 * q + i, k));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[kf][e] = g[2 * e] | (g[2 * e + 1] << 16);
      }
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bf[nf] = *reinterpret_cast<const u32x4_t*>(s_b[hs] + slice_off(16 * nf + lr, 8 * q));
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[kf][nf] = mfma_16x16x32(a[kf], bf[nf], acc[kf][nf]);
    }
  }
  // (the codebook was written before the first barrier: r >= 1)
  if (!k_in) return;

  // epilogue: tile kf gives this lane columns kw + 16q + 4kf + v, v = 0..3,
  // of row n0 + 16nf + lr: columns kw + 16q + c, c = 4kf + v, in order
  const float mu = *W.mu;
#pragma unroll
  for (int nf = 0; nf < 4; ++nf) {
    const int64_t n = n0 + 16 * nf + lr;
    if (n >= N) continue;
    const float cp = decode_constant(ee[nf], __uint_as_float(ss[nf]), mu);
    uint32_t o[8];
#pragma unroll
    for (int kf = 0; kf < 4; ++kf) {
      const uint32_t c16 = (cw[nf][kf >> 1] >> (16 * (kf & 1))) & 0xffffu;  // codes of columns 4kf .. +3
      float m[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t code = (c16 >> (4 * v)) & 15u;
        const float w_hat = bf16lo(pack_bf16x2(__fmul_rn(s_q[code], cp), 0.0f));
        m[v] = __fadd_rn(w_hat, __fmul_rn(scale, acc[kf][nf][v]));
      }
      o[2 * kf] = pack_out<F16>(m[0], m[1]);
      o[2 * kf + 1] = pack_out<F16>(m[2], m[3]);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + n * K + kw + 16 * q);
    dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
  }
}

}  // namespace

hipError_t launch_merge(const Nf4View& W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                        uint16_t* out, bool out_f16, hipStream_t st) {
  const int64_t col_tiles = (W.K + kMergeCols - 1) / kMergeCols;
  const int64_t row_tiles = (W.N + kMergeRows - 1) / kMergeRows;
  const int64_t grid = col_tiles * row_tiles;
  if (grid == 0) return hipSuccess;
  return out_f16 ? timed_launch(kKernMerge, merge_kernel<true>, dim3((unsigned)grid), dim3(kMergeThreads), st, W,
                                A, B, (int)r, scale, out, (uint32_t)col_tiles, codebook())
                 : timed_launch(kKernMerge, merge_kernel<false>, dim3((unsigned)grid), dim3(kMergeThreads), st, W,
                                A, B, (int)r, scale, out, (uint32_t)col_tiles, codebook());
}

}  // namespace qnf4
