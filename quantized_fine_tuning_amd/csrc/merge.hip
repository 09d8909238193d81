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
// merge_kernel: a grid of about two workgroups (4 waves each) per compute
// unit.  The weight is cut into tiles of 64 rows x 256 columns; workgroup b
// keeps one column strip (b % col_tiles) and walks down its row tiles
// (b / col_tiles, then every g-th), so the strip's slice of A is copied into
// LDS once when r <= 64 (once per tile and 64-rank chunk above that), and the
// next tile's codes, constants and B rows are requested before the current
// tile's epilogue, so that their latency overlaps its arithmetic and stores.
//   * The rank-r product D[k][n] = Σ_j A[j][k]·B[n][j] runs in chunks of 64
//     ranks (two slices of 32): the A slices (32 x 256 each) copied from
//     memory straight into LDS, row-major, their MFMA fragments (8
//     consecutive ranks of one column) gathered with 2-byte reads; the B
//     slices (64 x 32) through registers (two-byte loads: B's rows need not
//     be aligned), whose rows are fragments already.
//   * Wave w owns columns kw = k0 + 64w .. +63 (one NF4 block of each row)
//     against all 64 rows: 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  The
//     MFMA row i of column tile kf stands for column kw + 32(kf / 2) +
//     8(i / 4) + 4(kf % 2) + i % 4, so that lane (l % 16, q = l / 16), which
//     receives MFMA rows 4q .. 4q+3 of every tile, ends with the 8-column
//     pieces q and q + 4 of its row: each of the row's two 16-byte store
//     instructions writes 64 contiguous bytes of it.
//   * Codes: lane (l % 16, q) loads the 32 code bytes of row 16q + l % 16's
//     block; the wave passes them round through LDS (a dword-swizzled 2 KB
//     per wave), each lane reading the 4 + 4 bytes of its pieces in each of
//     its 4 rows.
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int kMergeRows = 64, kMergeCols = 256, kMergeThreads = 256;
constexpr int kMergeChunk = 64;            // ranks per chunk (two slices of 32)
constexpr int kMergeWorkgroups = 2 * 256;  // about two per compute unit

// Byte offset of element (row, j) of a B slice (64-byte rows, 16-byte chunk c
// of row `row` at physical chunk c ^ ((row >> 1) & 3)): the 8 lanes of one
// 16-byte fragment read (rows 0..7 of a tile) hit distinct banks.
__device__ __forceinline__ uint32_t slice_off(int row, int j) {
  return (uint32_t)(row * 64 + (((j >> 3) ^ ((row >> 1) & 3)) << 4) + 2 * (j & 7));
}
// Byte offset of element (j, k) of an A slice (512-byte rows; in the rows of
// odd 8-row groups the 64-byte quarters swap in pairs, columns XOR 32): a
// gather of one rank by a quarter-wave reads 8 dwords within one 16-bank
// half, and the other quarter-wave of the half-wave (rows 8 further) the
// same dwords of the other half.
__device__ __forceinline__ uint32_t aslice_off(int j, int k) {
  return (uint32_t)(j * 512 + 2 * (k ^ ((j & 8) << 2)));
}
// the column (within the wave's 64) that MFMA row i of column tile kf stands for
__device__ __forceinline__ int tile_col(int kf, int i) {
  return 32 * (kf >> 1) + 8 * (i >> 2) + 4 * (kf & 1) + (i & 3);
}
// Dword d of row R's 32 code bytes in a wave's LDS area: 8 dwords per row,
// XOR 2((R / 4) % 4), so that the reads of one dword position by the 32
// lanes of a half-wave (rows R = 16nf + l % 16, positions q, q ^ 1) fall on
// distinct banks.
__device__ __forceinline__ uint32_t code_off(int R, int d) {
  return (uint32_t)(4 * (8 * R + (d ^ (2 * ((R >> 2) & 3)))));
}

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

// what a lane needs of one row tile besides the product: codes of its 16
// columns in each of its 4 rows, the e4m3 constant and group scale of one
// row (the 4 lanes of a row pass them round), and its 8 B values of each
// slice of the chunk
struct TileRegs {
  u32x4_t cr[2];    // the 32 code bytes of row 16q + l % 16
  uint32_t e1, s1;  // constant and group scale of row 16q + l % 16 (shared by shuffles)
  u32x4_t hb[2];  // B row t / 4, ranks 8(t % 4) .. +7 of the chunk's two slices
};

template <bool F16>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(Nf4View W, const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B, int r,
                                                              float scale, uint16_t* __restrict__ out,
                                                              uint32_t col_tiles, uint32_t row_tiles,
                                                              uint32_t row_step, Codebook cb) {
  __shared__ __attribute__((aligned(1024))) char s_a[2][32 * kMergeCols * 2];  // A slices [32 j][256 k]
  __shared__ __attribute__((aligned(16))) char s_b[2][kMergeRows * 64];       // B slices [64 n][32 j]
  __shared__ __attribute__((aligned(16))) uint32_t s_code[4][64 * 8];  // per wave: 64 rows x 32 code bytes
  __shared__ float s_q[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const int64_t N = W.N, K = W.K;
  const int64_t k0 = (int64_t)(blockIdx.x % col_tiles) * kMergeCols;
  const int64_t kw = k0 + 64 * wave;  // this wave's block column
  const bool k_in = kw < K;
  const int64_t kpr = K / kBlock;     // blocks per row
  const float mu = *W.mu;

  const rsrc_t rc = make_rsrc(W.codes, N * K / 2);
  const rsrc_t re = make_rsrc(W.e, N * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t ra = make_rsrc(A, (int64_t)r * K * 2);
  const rsrc_t rb = make_rsrc(B, N * r * 2);
  // A copy: wave instruction c of a slice fills rows 2(4w + c) and +1 (1 KB);
  // lane i lands at byte 16i of them: row 2(4w + c) + i / 32, physical piece
  // i % 32, which holds logical columns 8((i % 32) ^ (row & 8 ? 4 : 0))
  const int crow0 = lane >> 5, cpiece = lane & 31;
  // B: thread t loads row t / 4, ranks 8(t % 4) .. +7 of each slice
  const int bnl = tid >> 2, bjc = 8 * (tid & 3);

  auto load_a = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int j0 = c0 + 32 * hs;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int jj = 2 * (4 * wave + c) + crow0;
        const int kc = 8 * (cpiece ^ ((jj & 8) ? 4 : 0));
        const bool ok = j0 + jj < r && k0 + kc < K;
        buf_load_lds16(ra, s_a[hs] + 1024 * (4 * wave + c),
                       ok ? (uint32_t)(((int64_t)(j0 + jj) * K + k0 + kc) * 2) : 0x7fffffffu, 0u);
      }
    }
  };
  // (rows of B are 16-byte aligned when r % 8 == 0: one 16-byte load per
  // slice; otherwise eight 2-byte loads)
  const bool b_wide = (r & 7) == 0;
  auto load_b = [&](TileRegs& t, int64_t n0, int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int j0 = c0 + 32 * hs + bjc;
      if (b_wide) {
        t.hb[hs] = buf_load16(rb, j0 < r ? (uint32_t)(((n0 + bnl) * r + j0) * 2) : 0x7fffffffu, 0u);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = buf_load2(rb, j0 + e < r ? (uint32_t)(((n0 + bnl) * r + j0 + e) * 2) : 0x7fffffffu, 0u);
#pragma unroll
        for (int e = 0; e < 4; ++e) t.hb[hs][e] = (h[2 * e] & 0xffffu) | (h[2 * e + 1] << 16);
      }
    }
  };
  // the block's codes and constants of row 16q + l % 16; rows past N read
  // zero, a wave past K loads nothing
  auto load_codes = [&](TileRegs& t, int64_t n0) __attribute__((always_inline)) {
    const int64_t n = n0 + 16 * q + lr;
    const int64_t b = n * kpr + kw / kBlock;
    const bool ok = k_in && n < N;
    const uint32_t co = ok ? (uint32_t)(b * (kBlock / 2)) : 0x7fffffffu;
    t.cr[0] = buf_load16(rc, co, 0u);
    t.cr[1] = buf_load16(rc, co, 16u);
    t.e1 = buf_load1(re, ok ? (uint32_t)b : 0x7fffffffu, 0u);
    t.s1 = buf_load4(rs, ok ? (uint32_t)((b / kDqBlock) * 4) : 0x7fffffffu, 0u);
  };

  uint32_t rt = blockIdx.x / col_tiles;
  TileRegs cur;
  load_codes(cur, (int64_t)rt * kMergeRows);
  load_b(cur, (int64_t)rt * kMergeRows, 0);
  load_a(0);
  if (tid < 16) s_q[tid] = cb.q[tid];
  wait_vmem();  // this wave's copies into LDS have landed (the barrier below publishes them)

  for (; rt < row_tiles; rt += row_step) {
    const int64_t n0 = (int64_t)rt * kMergeRows;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < r; c0 += kMergeChunk) {
      if (c0 > 0) {  // r > 64: this chunk's A and B
        __syncthreads();  // the previous chunk's reads are done
        load_a(c0);
        load_b(cur, n0, c0);
        wait_vmem();
      }
      __syncthreads();  // s_b free (previous chunk or tile read it); A copies visible
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) *reinterpret_cast<u32x4_t*>(s_b[hs] + slice_off(bnl, bjc)) = cur.hb[hs];
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
          for (int i = 0; i < 8; ++i)
            g[i] = *reinterpret_cast<const uint16_t*>(s_a[hs] + aslice_off(8 * q + i, k));
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

    // the next tile's registers (and, for r > 64, its first A chunk once
    // every wave is done with this tile's)
    const uint32_t rn = rt + row_step;
    TileRegs nxt;
    if (rn < row_tiles) {
      if (r > kMergeChunk) {
        __syncthreads();
        load_a(0);
      }
      load_codes(nxt, (int64_t)rn * kMergeRows);
      load_b(nxt, (int64_t)rn * kMergeRows, 0);
    }

    // epilogue: tile kf gives this lane columns 32(kf / 2) + 8q + 4(kf % 2) +
    // v, v = 0..3, of the wave's 64 in row n0 + 16nf + lr: pieces q (kf = 0,
    // 1) and q + 4 (kf = 2, 3), columns in order
    if (k_in) {
      // the codes round the wave: row 16q + lr's 8 dwords in, then per row
      // the dwords q (columns 8q .. +7) and 4 + q (columns 32 + 8q .. +7)
      uint32_t* sc = s_code[wave];
      const int Rme = 16 * q + lr;
#pragma unroll
      for (int d = 0; d < 8; ++d) sc[code_off(Rme, d) / 4] = cur.cr[d >> 2][d & 3];
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      uint32_t cq[4][2];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        cq[nf][0] = sc[code_off(16 * nf + lr, q) / 4];
        cq[nf][1] = sc[code_off(16 * nf + lr, 4 + q) / 4];
      }
      // row 16nf + lr's constants are lane (lr, nf)'s (shuffled while every
      // lane is active)
      uint32_t e[4], sg[4];
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        e[nf] = (uint32_t)__shfl((int)cur.e1, lr + 16 * nf, 64);
        sg[nf] = (uint32_t)__shfl((int)cur.s1, lr + 16 * nf, 64);
      }
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int64_t n = n0 + 16 * nf + lr;
        if (n >= N) continue;
        const float cp = decode_constant(e[nf], __uint_as_float(sg[nf]), mu);
        uint32_t o[8];
#pragma unroll
        for (int kf = 0; kf < 4; ++kf) {
          const uint32_t c16 = (cq[nf][kf >> 1] >> (16 * (kf & 1))) & 0xffffu;  // 4 columns of tile kf
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
        uint16_t* dst = out + n * K + kw + 8 * q;
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4_t*>(dst + 32) = u32x4_t{o[4], o[5], o[6], o[7]};
      }
    }
    if (rn < row_tiles && r > kMergeChunk) wait_vmem();  // the A copy above
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_merge(const Nf4View& W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                        uint16_t* out, bool out_f16, hipStream_t st) {
  const int64_t col_tiles = (W.K + kMergeCols - 1) / kMergeCols;
  const int64_t row_tiles = (W.N + kMergeRows - 1) / kMergeRows;
  if (col_tiles == 0 || row_tiles == 0) return hipSuccess;
  // workgroups per column strip: all strips get the same number, each
  // walking its row tiles with that stride
  const int64_t per_strip = std::max<int64_t>(1, std::min<int64_t>(row_tiles, kMergeWorkgroups / col_tiles));
  const unsigned grid = (unsigned)(col_tiles * per_strip);
  return out_f16 ? timed_launch(kKernMerge, merge_kernel<true>, dim3(grid), dim3(kMergeThreads), st, W, A, B,
                                (int)r, scale, out, (uint32_t)col_tiles, (uint32_t)row_tiles,
                                (uint32_t)per_strip, codebook())
                 : timed_launch(kKernMerge, merge_kernel<false>, dim3(grid), dim3(kMergeThreads), st, W, A, B,
                                (int)r, scale, out, (uint32_t)col_tiles, (uint32_t)row_tiles,
                                (uint32_t)per_strip, codebook());
}

}  // namespace qnf4
