// Forward product of the QLoRA linear layer for M > 16 tokens, gfx950:
//   Y[M, N] = X·Ŵᵀ + s·T·Bᵀ  =  [X | sT_hi | sT_lo] · [Ŵ | B | B]ᵀ
// (P1 §七 dataflow figure: the 4-bit base is dequantized to BF16 for the
// matmul and the LoRA path is added to the output.)
//
// Design
//   * 256x256 output tile per workgroup of 8 waves, two per SIMD: while one
//     wave of a SIMD issues MFMAs the other can issue its dequantization
//     arithmetic (within one wave the two largely serialize).
//   * Per 64-wide reduction step every wave dequantizes 32 of the tile's 256
//     weight rows into a shared bf16 tile Ŵ[n][k] in LDS; then wave (wm, wn)
//     multiplies token rows [128wm, +128) by weight rows [64wn, +64): 64
//     v_mfma_f32_16x16x32_bf16 per wave and step, operands read from LDS.
//   * Dequantization goes through a per-row table: lane t < 32 writes the 16
//     values RNE_bf16(fl32(q_j * c')) of row t to LDS, and every code is one
//     2-byte table read (bit-identical to multiplying per element, since the
//     value depends only on code and row).  Lane l reads rows 8q + (l >> 3),
//     k = 8(l & 7) + 0..7: the 8 lanes of one row hit its table, and the 4
//     rows of each half-wave (served in one LDS cycle) hit 4 different
//     groups of 8 of the 32 banks, so lookups never conflict.
//   * Tiles are stored with 16-byte chunks XOR-swizzled by row (xswz) so that
//     MFMA operand reads of 8 rows cover the 32 LDS banks once.
//   * The X tile of the next step is copied straight into LDS; the weight
//     data (packed codes, e4m3 bytes, group scales) of the step after is
//     loaded into registers at the top of an iteration and stored to LDS at
//     its end, so no loaded register lives across iterations.  The MFMAs of
//     step s are interleaved in issue order with the dequantization of step
//     s+1 into the other Ŵ buffer, in the first half of the step for one wave
//     of each SIMD and in the second half for the other.
//   * All operand reads are buffer loads whose resources end at the tensor's
//     last row, so ragged tiles read zeros without per-lane branches.
//   * The LoRA up-projection is 2*Rp/64 extra reduction steps whose A operand
//     is the bf16 hi/lo split of s·T and whose B operand is the padded copy
//     B2 = [B | 0 | B | 0] ([N, 2Rp] bf16), both copied straight into LDS.
//   * Workgroups are mapped to tiles so that each XCD (workgroup id mod 8)
//     walks a contiguous run of a grouped tile order (4 M-tiles per group):
//     the ~32 workgroups resident on one XCD share X and code rows in its L2.
#include <type_traits>

#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TN = 256, KSTEP = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// A tile row = 64 bf16 = eight 16-byte chunks; chunk c of row r is stored at
// physical chunk c ^ (r & 7).  LDS has 32 banks of 4 bytes and serves a
// 16-byte read for 8 lanes per cycle: an MFMA operand read gives those 8
// lanes 8 consecutive rows, whose chunks then cover the 32 banks once.
__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int LSTEPS>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                               int64_t M, const uint16_t* __restrict__ sT,
                                                               const uint16_t* __restrict__ B2,
                                                               int64_t Rp, void* __restrict__ Y,
                                                               int y_bf16, int tiles_m, int tiles_n,
                                                               Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sx0[TM * 128], sx1[TM * 128];  // A tiles: X, then sT
  __shared__ __attribute__((aligned(16))) char sw[2][TN * 128];  // B tiles: Ŵ, then B2
  // per wave: tables of its 32 rows (row t at 32(t % 8) + 256(t / 8)), the
  // packed codes of its rows (32 bytes each) and, per row, the dword holding
  // its e4m3 byte and its group scale; code data double-buffered by step
  __shared__ __attribute__((aligned(256))) char slut[kWaves][32 * 32];
  __shared__ __attribute__((aligned(16))) char scode[2][kWaves][32 * 32];
  __shared__ __attribute__((aligned(16))) uint32_t sconst[2][kWaves][2][32];
  __shared__ float sq[16];
  int tmi, tni;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tmi, tni)) return;
  if (threadIdx.x < 16) sq[threadIdx.x] = cb.q[threadIdx.x];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t K = W.K, N = W.N;
  const int64_t m0 = (int64_t)tmi * TM, n0 = (int64_t)tni * TN;
  const int ksteps = (int)(K / KSTEP);
  const uint32_t kpr = (uint32_t)(K / kBlock);  // blocks per weight row
  const float mu = *W.mu;

  // Resources start at this tile's first row and end at the tensor's last
  // row: rows past M or N read as zero.  (Rows past M only feed output rows
  // past M, rows past N only output columns past N; neither is stored.)
  const rsrc_t rx = make_rsrc(X + m0 * K, (M - m0) * K * 2);
  const rsrc_t rt = make_rsrc(sT + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t rc = make_rsrc(W.codes + n0 * (K / 2), (N - n0) * (K / 2));
  const rsrc_t re = make_rsrc(W.e + n0 * kpr, (N - n0) * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rb = make_rsrc(B2 + n0 * 2 * Rp, (N - n0) * 2 * Rp * 2);

  // X tile, copied straight into LDS: thread τ moves 16 bytes of rows
  // 64c + (τ >> 3), c = 0..3, into physical chunk τ & 7, so it fetches
  // logical chunk (τ & 7) ^ ((τ >> 3) & 7) (row & 7 does not depend on c).
  // LDS offset 64c*128 + 16τ: each wave's copy is 1 KB contiguous.
  const int xlch = (tid & 7) ^ ((tid >> 3) & 7);
  const uint32_t vx = (uint32_t)(((tid >> 3) * K + 8 * xlch) * 2);
  const uint32_t x_gstride = (uint32_t)(64 * K * 2);
  // (written as assembly: the compiler then inserts no wait for these copies
  // in front of the LDS reads of the step; the wait before the step's
  // closing barrier is explicit)
  const i32x4_t rxw = rsrc_words(X + m0 * K, (M - m0) * K * 2);
  auto copy_x = [&](char* t, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dma_lds16(rxw, t + 64 * c * 128 + 1024 * wave, vx + c * x_gstride, (uint32_t)s * 128u);
  };
  auto sxb = [&](int i) { return i ? sx1 : sx0; };
  // LoRA tiles (sT rows, B2 rows) copied straight into LDS: wave w copies rows
  // 32w + 8c + (i >> 3), c = 0..3, lane i into physical chunk i & 7, so it
  // fetches logical chunk (i & 7) ^ (i >> 3).
  const int llch = (lane & 7) ^ (lane >> 3);
  const uint32_t vl = (uint32_t)(((32 * wave + (lane >> 3)) * 2 * Rp + 8 * llch) * 2);
  const uint32_t l_gstride = (uint32_t)(8 * 2 * Rp * 2);
  auto copy_lora = [&](rsrc_t r, char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      buf_load_lds16(r, t + (32 * wave + 8 * c) * 128, vl, c * l_gstride + (uint32_t)l * 128u);
  };

  // Weight data of the wave's rows [32w, 32w+32) for step t: lane l loads 16
  // code bytes of row l/2 (half l%2); lane l < 32 the dword holding the e4m3
  // byte of row l and that row's group scale (lanes >= 32 repeat them).
  const uint32_t vcd = (uint32_t)((32 * wave + (lane >> 1)) * (K / 2) + (lane & 1) * 16);
  const int crow = 32 * wave + (lane & 31);
  const uint32_t ve_me = (uint32_t)crow * kpr;
  const uint32_t blk_me = (uint32_t)(n0 + crow) * kpr;
  struct WRegs {
    u32x4_t c;
    uint32_t e, s;
  };
  auto load_w = [&](WRegs& r, int t) __attribute__((always_inline)) {
    r.c = buf_load16(rc, vcd, (uint32_t)t * 32u);
    r.e = buf_load4(re, (ve_me + (uint32_t)t) & ~3u, 0u);
    r.s = buf_load4(rs, ((blk_me + (uint32_t)t) / kDqBlock) * 4u, 0u);
  };
  auto store_w = [&](int slot, const WRegs& r) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4_t*>(scode[slot][wave] + 16 * lane) = r.c;
    if (lane < 32) {
      sconst[slot][wave][0][lane] = r.e;
      sconst[slot][wave][1][lane] = r.s;
    }
  };

  // Dequantization of step t (weight data in slot) into the tile `dst`.
  char* lut = slut[wave];
  const int dr = lane >> 3, dc = lane & 7;  // row 8q + dr of the wave, k-chunk dc
  const uint32_t lut_lane = lds_offset(lut) + (uint32_t)dr * 32u;
  auto build_table = [&](int t, int slot) __attribute__((always_inline)) {
    if (lane < 32) {
      const uint32_t e = (sconst[slot][wave][0][lane] >> (8 * ((ve_me + (uint32_t)t) & 3u))) & 0xffu;
      const float cp = decode_constant(e, __uint_as_float(sconst[slot][wave][1][lane]), mu);
      u32x4_t t0, t1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        t0[p] = pack_bf16x2(__fmul_rn(sq[2 * p], cp), __fmul_rn(sq[2 * p + 1], cp));
        t1[p] = pack_bf16x2(__fmul_rn(sq[8 + 2 * p], cp), __fmul_rn(sq[9 + 2 * p], cp));
      }
      char* row = lut + 32 * (lane & 7) + 256 * (lane >> 3);
      *reinterpret_cast<u32x4_t*>(row) = t0;
      *reinterpret_cast<u32x4_t*>(row + 16) = t1;
    }
  };
  // rows 8q + dr: the code dword of k-chunk dc, its 8 table lookups, one
  // 16-byte store of 8 consecutive bf16
  auto dequant_group = [&](int slot, char* dst, int q) __attribute__((always_inline)) {
    const uint32_t w =
        *reinterpret_cast<const uint32_t*>(scode[slot][wave] + (8 * q + dr) * 32 + dc * 4);
    const uint32_t tab = lut_lane + 256u * (uint32_t)q;  // 32-byte aligned
    u32x4_t o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      u16x2_t v;
      v.x = lds_read_u16(tab | code_x2(w, 8 * p));
      v.y = lds_read_u16(tab | code_x2(w, 8 * p + 4));
      o[p] = __builtin_bit_cast(uint32_t, v);
    }
    *reinterpret_cast<u32x4_t*>(dst + xswz(32 * wave + 8 * q + dr, dc)) = o;
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // MFMA group g (0..15) of a step: k-half ks = g / 8, token block i = g % 8;
  // B fragments of the k-half are read at its first group.
  const int arow = 128 * wm + lr, brow = 64 * wn + lr;
  u32x4_t bfr[4];
  auto mfma_group = [&](const char* xa, const char* wb, int g) __attribute__((always_inline)) {
    const int ks = g >> 3, i = g & 7;
    if (i == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const u32x4_t*>(wb + xswz(brow + 16 * j, 2 * kq + ks));
    }
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(xa + xswz(arow + 16 * i, 2 * kq + ks));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(a, bfr[j], acc[i][j]);
  };
  auto mfma_step = [&](const char* xa, const char* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 16; ++g) mfma_group(xa, wb, g);
  };
  // The MFMAs of one step interleaved with the dequantization of step t:
  // table build next to the first groups, one row group of lookups every
  // three MFMA groups.
  // The two waves of a SIMD (w and w + 4, i.e. wm = 0 and 1) dequantize in
  // different halves of the step (phase P = wm): while one issues table
  // arithmetic and lookups, the other issues MFMAs.  Both instances keep the
  // same barrier sequence.
  auto mfma_step_dequant = [&](auto P, const char* xa, const char* wb, int t, int slot, char* dst)
      __attribute__((always_inline)) {
    constexpr int g0 = decltype(P)::value ? 8 : 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      mfma_group(xa, wb, g);
      if (g == g0) build_table(t, slot);
      if (g > g0 && g <= g0 + 4) dequant_group(slot, dst, g - g0 - 1);
    }
  };

  // prologue: X and weight data of step 0, weight data of step 1 (K >= 64,
  // so step 0 is a weight step); dequantize step 0
  {
    WRegs w0, w1;
    copy_x(sx0, 0);
    load_w(w0, 0);
    load_w(w1, 1);
    store_w(0, w0);
    store_w(1, w1);
  }
  wait_vmem();
  __syncthreads();
  build_table(0, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) dequant_group(0, sw[0], q);
  __syncthreads();

  // Weight steps 0 .. ksteps-2: copy X of step s+1 into the other X buffer
  // and load the weight data of step s+2 into registers, issue the MFMAs of
  // step s interleaved with the dequantization of step s+1 into the other Ŵ
  // buffer, then store the weight data into slot s % 2 (both buffers last
  // read in the previous iteration).  (Weight data of step ksteps may be
  // loaded: its reads stay inside the buffers or return zeros, and it is not
  // used.)  One step per iteration and no other loop carrying the
  // accumulators: anything else makes the register allocator shuffle or
  // spill them.  The loop is instantiated once per phase.
  auto iter = [&](auto P, int s, const char* xa, char* xn) __attribute__((always_inline)) {
    WRegs wr;
    copy_x(xn, s + 1);
    load_w(wr, s + 2);
    mfma_step_dequant(P, xa, sw[s & 1], s + 1, (s + 1) & 1, sw[(s + 1) & 1]);
    store_w(s & 1, wr);
    wait_vmem();
    __syncthreads();
  };
  auto main_loop = [&](auto P) __attribute__((always_inline)) {
#pragma unroll 1
    for (int s = 0; s + 1 < ksteps; ++s) iter(P, s, sxb(s & 1), sxb((s + 1) & 1));
  };
  if (wm == 0)
    main_loop(std::integral_constant<int, 0>());
  else
    main_loop(std::integral_constant<int, 1>());
  // Last weight step, copying LoRA step 0 (sT and B2 tiles) into the other
  // buffers; then the LoRA steps, unrolled.
  copy_lora(rt, sxb(ksteps & 1), 0);
  copy_lora(rb, sw[ksteps & 1], 0);
  mfma_step(sxb((ksteps - 1) & 1), sw[(ksteps - 1) & 1]);
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int l = 0; l < LSTEPS; ++l) {
    const int s = ksteps + l;
    if (l + 1 < LSTEPS) {
      copy_lora(rt, sxb((s + 1) & 1), l + 1);
      copy_lora(rb, sw[(s + 1) & 1], l + 1);
    }
    mfma_step(sxb(s & 1), sw[s & 1]);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane holds rows 128wm + 16i + 4kq + v of column 64wn + 16j + lr.
  // The row/column bases go through an empty asm so that their address
  // arithmetic is not hoisted above the main loop (it would stay live there).
  int row0 = 128 * wm + 4 * kq, col0 = 64 * wn + lr;
  asm volatile("" : "+v"(row0), "+v"(col0));
  const bool full = (m0 + TM <= M) && (n0 + TN <= N);
  if (y_bf16) {
    uint16_t* Yb = static_cast<uint16_t*>(Y) + (m0 + row0) * N + n0 + col0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, n = n0 + col0 + 16 * j;
          if (full || (m < M && n < N))
            Yb[(16 * i + v) * N + 16 * j] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xffffu);
        }
  } else {
    float* Yf = static_cast<float*>(Y) + (m0 + row0) * N + n0 + col0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, n = n0 + col0 + 16 * j;
          if (full || (m < M && n < N)) Yf[(16 * i + v) * N + 16 * j] = acc[i][j][v];
        }
  }
}

// B2[n][j] = B[n][j mod Rp] for (j mod Rp) < r, else 0;  [N, 2Rp] bf16.
__global__ void pad_lora_b_kernel(const uint16_t* __restrict__ B, int64_t N, int r, int64_t Rp,
                                  uint16_t* __restrict__ B2) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * 2 * Rp) return;
  const int64_t n = idx / (2 * Rp), j = (idx % (2 * Rp)) % Rp;
  B2[idx] = j < r ? B[n * r + j] : (uint16_t)0;
}

}  // namespace

hipError_t launch_pad_lora_b(const uint16_t* B, int64_t N, int32_t r, int64_t Rp, uint16_t* B2,
                             hipStream_t st) {
  const int64_t n2 = N * 2 * Rp;
  pad_lora_b_kernel<<<(unsigned)((n2 + 255) / 256), 256, 0, st>>>(B, N, r, Rp, B2);
  return hipGetLastError();
}

hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B, int32_t r, int64_t Rp, uint16_t* B2, void* Y,
                           bool y_bf16, hipStream_t st) {
  hipError_t e = launch_pad_lora_b(B, W.N, r, Rp, B2, st);
  if (e != hipSuccess) return e;
  const int tm = (int)((M + TM - 1) / TM), tn = (int)((W.N + TN - 1) / TN);
  const unsigned grid = tile_grid(tm, tn);
  const int yb = y_bf16 ? 1 : 0;
  switch (2 * Rp / KSTEP) {
#define QNF4_FWD_CASE(LS)                                                                   \
  case LS:                                                                                  \
    return timed_launch(kKernFwdGemm, fwd_gemm_kernel<LS>, dim3(grid), dim3(kThreads), st, W, X, M, \
                        (const uint16_t*)sT, (const uint16_t*)B2, Rp, Y, yb, tm, tn, codebook());
    QNF4_FWD_CASE(1)
    QNF4_FWD_CASE(2)
    QNF4_FWD_CASE(3)
    QNF4_FWD_CASE(4)
    QNF4_FWD_CASE(5)
    QNF4_FWD_CASE(6)
    QNF4_FWD_CASE(7)
    QNF4_FWD_CASE(8)
#undef QNF4_FWD_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qnf4
