// Input gradient of the QLoRA linear layer, gfx950:
//   dX[M, K] = dY·Ŵ + s·U·A  =  [dY | sU_hi | sU_lo] · [Ŵ ; A ; A]
// (P1 简化版 and P2 §4.4: the gradient passes through the dequantized frozen
// weight; U = dY·B is the LoRA path's input gradient.)
//
// The reduction runs over the weight's rows n while the codes are contiguous
// along k, so the dequantized weight has to be transposed on its way to the
// MFMA B operand.  Design:
//   * 256x256 output tile per workgroup (token rows x input features) of 8
//     waves, two per SIMD, so that one wave's dequantization arithmetic can
//     issue while the other wave's MFMAs run.
//   * Per 64-row reduction step every wave dequantizes 32 of the tile's 256
//     columns (half an NF4 block column) for all 64 weight rows into a shared
//     transposed bf16 tile Ŵᵀ[k][n] in LDS; then wave (wm, wk) multiplies
//     token rows [128wm, +128) by columns [64wk, +64): 64
//     v_mfma_f32_16x16x32_bf16 per wave and step, operands read from LDS.
//   * Dequantization goes through a per-row table: for each weight row of
//     the step one lane writes the 16 values RNE_bf16(fl32(q_j * c')) (its
//     block's scaled codebook) to LDS; lane (rg, cg) then owns rows
//     8rg..8rg+7 by columns 4cg..4cg+3 of the wave's slice, each code one
//     2-byte table read, and packs 8 consecutive rows of one column into one
//     16-byte store: the values come out already transposed.  Table slots,
//     tile swizzles and lane maps are chosen so that lookups, stores and
//     fragment reads are free of LDS bank conflicts (32 banks of 4 bytes).
//   * The dY tile of the next step is copied straight into LDS; the weight
//     data of the step after is loaded into registers at the top of an
//     iteration and stored to LDS at its end.  The MFMAs of step s are
//     interleaved in issue order with the dequantization of step s+1 into the
//     other Ŵᵀ buffer, in the first half of the step for one wave of each
//     SIMD and in the second half for the other.  Rows past N get an all-zero
//     table.
//   * The LoRA term is 2*Rp/64 extra steps with A = [sU_hi | sU_lo] and B from
//     AT2[k][j] = A[j mod Rp][k] (a transposed, padded copy of A), both
//     copied straight into LDS.
#include <type_traits>

#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TK = 256, NSTEP = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// dY tile (token rows, 64 n each): chunk c of row r at physical c ^ (r & 7);
// a fragment read gives the 8 lanes of one LDS cycle 8 consecutive rows.
__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}
// Ŵᵀ tile (k rows, 64 n each): chunk c of row r at physical
// c ^ ((r ^ (r >> 2)) & 7), distinct both for 8 consecutive rows (fragment
// reads) and for rows 4cg + c, cg = 0..7 (the dequantization stores).
__device__ __forceinline__ int wswz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 2)) & 7)) << 4);
}

template <int LSTEPS>
__global__ __launch_bounds__(kThreads, 1) void dx_gemm_kernel(Nf4View W, const uint16_t* __restrict__ dY,
                                                              int64_t M, const uint16_t* __restrict__ sU,
                                                              const uint16_t* __restrict__ AT2,
                                                              int64_t Rp, void* __restrict__ dX,
                                                              int dx_bf16, int tiles_m, int tiles_k,
                                                              Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sa0[TM * 128], sa1[TM * 128];  // A tiles: dY, then sU
  __shared__ __attribute__((aligned(16))) char sw[2][TK * 128];  // B tiles: Ŵᵀ, then AT2
  // per wave (all wave-private, so one buffer each): 64 row tables of 32
  // bytes, the 16 code bytes of each weight row for the wave's 32 columns,
  // and each table row's e4m3 byte and group scale
  __shared__ __attribute__((aligned(256))) char slut[kWaves][64 * 32];
  __shared__ __attribute__((aligned(16))) char scode[kWaves][64 * 16];
  __shared__ __attribute__((aligned(16))) uint32_t sconst[kWaves][2][64];
  int tmi, tki;
  if (!tile_of(blockIdx.x, tiles_m, tiles_k, tmi, tki)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int wm = wave >> 2, wk = wave & 3;
  const int rg = lane >> 3, cg = lane & 7;
  const int64_t K = W.K, N = W.N;
  const int64_t m0 = (int64_t)tmi * TM, k0 = (int64_t)tki * TK;
  const int64_t kw0 = k0 + 32 * wave;  // first column of this wave's dequantization slice
  const int nsteps = (int)((N + NSTEP - 1) / NSTEP);
  const uint32_t kpr = (uint32_t)(K / kBlock);
  const uint32_t kbw = (uint32_t)(kw0 / kBlock);  // the slice's block column
  const bool wave_cols_ok = kw0 < K;
  const float mu = *W.mu;

  const rsrc_t rdy = make_rsrc(dY + m0 * N, (M - m0) * N * 2);
  const rsrc_t rsu = make_rsrc(sU + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t rc = make_rsrc(W.codes, N * (K / 2));
  const rsrc_t re = make_rsrc(W.e, N * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rat = make_rsrc(AT2 + k0 * 2 * Rp, (K - k0) * 2 * Rp * 2);

  // dY tile, copied straight into LDS: thread τ moves 16 bytes of rows
  // 64c + (τ >> 3), c = 0..3, into physical chunk τ & 7: logical chunk
  // (τ & 7) ^ ((τ >> 3) & 7); each wave's copy is 1 KB contiguous.  (Written
  // as assembly: the compiler then inserts no wait for these copies in front
  // of the LDS reads of the step; the wait before the step's closing
  // barrier is explicit.)
  const int ylch = (tid & 7) ^ ((tid >> 3) & 7);
  const uint32_t vy = (uint32_t)(((tid >> 3) * N + 8 * ylch) * 2);
  const uint32_t y_gstride = (uint32_t)(64 * N * 2);
  const i32x4_t ryw = rsrc_words(dY + m0 * N, (M - m0) * N * 2);
  auto copy_y_part = [&](char* t, int s, int c) __attribute__((always_inline)) {
    dma_lds16(ryw, t + 64 * c * 128 + 1024 * wave, vy + c * y_gstride, (uint32_t)s * 128u);
  };
  auto copy_y = [&](char* t, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) copy_y_part(t, s, c);
  };
  auto sab = [&](int i) { return i ? sa1 : sa0; };
  // LoRA tiles copied straight into LDS: wave w copies rows 32w + 8c + (i >> 3),
  // lane i into physical chunk i & 7.  sU rows use xswz, AT2 rows wswz.
  const uint32_t vsu = (uint32_t)(((32 * wave + (lane >> 3)) * 2 * Rp + 8 * ((lane & 7) ^ (lane >> 3))) * 2);
  auto copy_su = [&](char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      buf_load_lds16(rsu, t + (32 * wave + 8 * c) * 128, vsu, c * (uint32_t)(8 * 2 * Rp * 2) + (uint32_t)l * 128u);
  };
  auto copy_at = [&](char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = 32 * wave + 8 * c + (lane >> 3);
      const int lch = (lane & 7) ^ ((row ^ (row >> 2)) & 7);
      buf_load_lds16(rat, t + (32 * wave + 8 * c) * 128, (uint32_t)((row * 2 * Rp + 8 * lch) * 2),
                     (uint32_t)l * 128u);
    }
  };

  // Weight data for step t: lane l loads the 16 code bytes of weight row
  // t*64 + l over the wave's 32 columns, the e4m3 byte of block (row, kbw)
  // and that block's group scale.
  const uint32_t vcode = (uint32_t)(lane * (K / 2) + kw0 / 2);
  const uint32_t code_sstride = (uint32_t)(NSTEP * (K / 2));
  struct WRegs {
    u32x4_t c;
    uint32_t e, s;
  };
  auto load_w = [&](WRegs& r, int t) __attribute__((always_inline)) {
    r.c = buf_load16(rc, vcode, (uint32_t)t * code_sstride);
    const uint32_t blk = ((uint32_t)t * NSTEP + lane) * kpr + kbw;
    r.e = buf_load1(re, blk, 0u);
    r.s = buf_load4(rs, (blk / kDqBlock) * 4u, 0u);
  };
  // The code bytes go to LDS transposed for the lanes that dequantize them:
  // the 2 bytes of column pair cg of row 8rg + i sit at byte 2i of 16-byte
  // slot 8rg + (cg ^ rg), so that lane (rg, cg) later reads its 8 rows'
  // codes with one 16-byte read.  Slot XOR: the writes of one pair index go
  // to 8 distinct slots of each 128-byte line, the reads of 8 consecutive
  // lanes to 8 distinct slots.
  const uint32_t code_wbase = (uint32_t)((lane >> 3) * 128 + ((lane >> 3) << 4) + 2 * (lane & 7));
  auto store_w = [&](const WRegs& r) __attribute__((always_inline)) {
    const uint32_t wb = opaque(code_wbase);
#pragma unroll
    for (int pc = 0; pc < 8; ++pc)
      *reinterpret_cast<uint16_t*>(scode[wave] + (wb ^ (uint32_t)(pc << 4))) =
          (uint16_t)(r.c[pc >> 1] >> (16 * (pc & 1)));
    sconst[wave][0][lane] = r.e;
    sconst[wave][1][lane] = r.s;
  };

  // Dequantization of step t (weight data in the wave's buffers) into dst.
  // The table of weight row 8rg + i sits at byte 256i + 32rg of the wave's
  // table area, so a lookup is (base of rg | 2*code) plus the constant 256i.
  // Lane t builds the table of row 8rg + i with rg = t0 + 2t1 + 4t3 and
  // i = t4 + 2t5 + 4t2 (t_b = bit b of t) and writes half t2 of it first:
  // the 8 lanes of each 16-byte write then cover a 128-byte line.
  const uint32_t lut_addr = lds_offset(slut[wave]);
  const uint32_t lut_rg = lut_addr + 32u * (uint32_t)rg;
  const int tb_rg = (lane & 3) | ((lane >> 1) & 4), tb_i = ((lane >> 4) & 3) | (lane & 4);
  const int tb_row = 8 * tb_rg + tb_i;
  const int tb_first = (lane >> 2) & 1;
  char* const tb_dst = slut[wave] + 256 * tb_i + 32 * tb_rg + 16 * tb_first;
  auto build_table = [&](int t) __attribute__((always_inline)) {
    const bool row_ok = wave_cols_ok && ((int64_t)t * NSTEP + tb_row < N);
    const float cp = decode_constant(sconst[wave][0][tb_row], __uint_as_float(sconst[wave][1][tb_row]), mu);
    u32x4_t t0, t1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      t0[p] = row_ok ? pack_bf16x2(__fmul_rn(cb.q[2 * p], cp), __fmul_rn(cb.q[2 * p + 1], cp)) : 0u;
      t1[p] = row_ok ? pack_bf16x2(__fmul_rn(cb.q[8 + 2 * p], cp), __fmul_rn(cb.q[9 + 2 * p], cp)) : 0u;
    }
    char* const d = opaque(tb_dst);
    *reinterpret_cast<u32x4_t*>(d) = tb_first ? t1 : t0;
    *reinterpret_cast<u32x4_t*>((char*)((uintptr_t)d ^ 16u)) = tb_first ? t0 : t1;
  };
  // The codes of rows 8rg..8rg+7, columns 4cg..4cg+3: row 2p in the low
  // half of dword p, row 2p + 1 in its high half.
  const int code_rslot = 8 * rg + (cg ^ rg);
  auto read_codes = [&]() __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4_t*>(scode[wave] + 16 * code_rslot);
  };
  // Column pair cp2 (columns 4cg + 2cp2, +1) of rows 8rg..8rg+7: 16
  // lookups, two 16-byte stores of 8 rows each.
  // Store address of column 4cg + c of the wave's slice, rows 8rg..8rg+7:
  // wswz(32w + 4cg + c, rg) = (st0 ^ 16c) + 128c.
  const uint32_t st0 = (uint32_t)((32 * wave + 4 * cg) * 128 + ((rg ^ cg ^ (4 * (cg & 1))) << 4));
  auto dequant_cols = [&](char* dst, int cp2, const u32x4_t& cw) __attribute__((always_inline)) {
    const uint32_t lb = opaque(lut_rg);
    uint16_t v[2][8];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int c = 2 * cp2 + cc;
        v[cc][2 * p] = lds_read_u16((lb | code_x2(cw[p], 4 * c)) + 256u * (2 * p));
        v[cc][2 * p + 1] = lds_read_u16((lb | code_x2(cw[p], 16 + 4 * c)) + 256u * (2 * p + 1));
      }
    // all 16 lookups are issued before the first result is used (one wait
    // instead of a chain of them); MFMAs, scalar and global-memory
    // instructions may still move across
    __builtin_amdgcn_sched_barrier(0x8 | 0x4 | 0x10);
    const uint32_t sb = opaque(st0);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int c = 2 * cp2 + cc;
      u32x4_t o;
#pragma unroll
      for (int p = 0; p < 4; ++p) o[p] = (uint32_t)v[cc][2 * p] | ((uint32_t)v[cc][2 * p + 1] << 16);
      *reinterpret_cast<u32x4_t*>(dst + ((sb ^ (uint32_t)(16 * c)) + 128u * c)) = o;
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // MFMA group g (0..15): n-half ks = g / 8, token block i = g % 8; the B
  // fragments of the half are read at its first group.
  // Fragment addresses: xswz(128wm + lr + 16i, 2kq + ks) = (a0 ^ 16ks) + 2048i
  // and wswz(64wk + lr + 16j, 2kq + ks) = (b0 ^ 16(ks + 4(j & 1))) + 2048j.
  const uint32_t a0 = (uint32_t)((128 * wm + lr) * 128 + (((2 * kq) ^ (lr & 7)) << 4));
  const uint32_t b0 = (uint32_t)((64 * wk + lr) * 128 + (((2 * kq) ^ ((lr ^ (lr >> 2)) & 7)) << 4));
  u32x4_t bfr[4];
  uint32_t abase = 0;
  auto mfma_group = [&](const char* ya, const char* wb, int g) __attribute__((always_inline)) {
    const int ks = g >> 3, i = g & 7;
    if (i == 0) {
      const uint32_t bb = opaque(b0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const u32x4_t*>(wb + ((bb ^ (uint32_t)(16 * (ks + 4 * (j & 1)))) + 2048u * j));
      abase = opaque(a0) ^ (uint32_t)(16 * ks);
    }
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(ya + abase + 2048u * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(a, bfr[j], acc[i][j]);
  };
  auto mfma_step = [&](const char* ya, const char* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 16; ++g) mfma_group(ya, wb, g);
  };
  // The two waves of a SIMD (w and w + 4, i.e. wm = 0 and 1) dequantize in
  // different halves of the step (phase P = wm): while one issues table
  // arithmetic and lookups, the other issues MFMAs.
  auto mfma_step_dequant = [&](auto P, const char* ya, const char* wb, int t, char* dst,
                               auto&& after_group) __attribute__((always_inline)) {
    constexpr int g0 = decltype(P)::value ? 8 : 0;
    u32x4_t cw;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      mfma_group(ya, wb, g);
      after_group(g);
      if (g == g0) {
        build_table(t);
        cw = read_codes();
      }
      if (g == g0 + 1 || g == g0 + 3) dequant_cols(dst, (g - g0 - 1) / 2, cw);
    }
  };

  // prologue: dY and weight data of step 0; dequantize step 0; weight data
  // of step 1
  {
    WRegs w0;
    copy_y(sa0, 0);
    load_w(w0, 0);
    store_w(w0);
  }
  wait_vmem();
  __syncthreads();  // dY and weight data of step 0
  build_table(0);
  {
    const u32x4_t cw = read_codes();
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) dequant_cols(sw[0], c2, cw);
  }
  {
    WRegs w1;
    load_w(w1, 1);
    store_w(w1);
  }
  __syncthreads();

  // Reduction steps 0 .. nsteps-2: copy dY of step s+1 into the other dY
  // buffer and load the weight data of step s+2, issue the MFMAs of step s
  // interleaved with the dequantization of step s+1 into the other Ŵᵀ
  // buffer, then store the loaded weight data (the weight buffers are
  // wave-private and were last read earlier in this iteration).  Weight data
  // of step nsteps may be loaded: its reads stay inside the buffers or
  // return zeros, and it is not used.  The loop is instantiated once per
  // phase.
  // Global reads queue behind one another in the compute unit's memory
  // pipeline, and a wave cannot issue past a read that does not fit: the
  // waves that dequantize first issue theirs at the top, the others one
  // after each of their first MFMA groups.
  auto main_loop = [&](auto P) __attribute__((always_inline)) {
    constexpr bool early = decltype(P)::value == 0;
#pragma unroll 1
    for (int s = 0; s + 1 < nsteps; ++s) {
      WRegs wr;
      if constexpr (early) {
        copy_y(sab((s + 1) & 1), s + 1);
        load_w(wr, s + 2);
      }
      mfma_step_dequant(P, sab(s & 1), sw[s & 1], s + 1, sw[(s + 1) & 1], [&](int g) {
        if constexpr (!early) {
          if (g < 4) copy_y_part(sab((s + 1) & 1), s + 1, g);
          if (g == 4) load_w(wr, s + 2);
        }
      });
      store_w(wr);
      wait_vmem();
      __syncthreads();
    }
  };
  if (wm == 0)
    main_loop(std::integral_constant<int, 0>());
  else
    main_loop(std::integral_constant<int, 1>());
  // last reduction step, copying LoRA step 0 (sU and AT2 tiles) into the
  // other buffers; then the LoRA steps, unrolled
  copy_su(sab(nsteps & 1), 0);
  copy_at(sw[nsteps & 1], 0);
  mfma_step(sab((nsteps - 1) & 1), sw[(nsteps - 1) & 1]);
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int l = 0; l < LSTEPS; ++l) {
    const int s = nsteps + l;
    if (l + 1 < LSTEPS) {
      copy_su(sab((s + 1) & 1), l + 1);
      copy_at(sw[(s + 1) & 1], l + 1);
    }
    mfma_step(sab(s & 1), sw[s & 1]);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane holds rows 128wm + 16i + 4kq + v of column k0 + 64wk + 16j + lr
  int row0 = 128 * wm + 4 * kq, col0 = 64 * wk + lr;
  asm volatile("" : "+v"(row0), "+v"(col0));
  const bool full = (m0 + TM <= M) && (k0 + TK <= K);
  if (dx_bf16) {
    uint16_t* D = static_cast<uint16_t*>(dX) + (m0 + row0) * K + k0 + col0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, k = k0 + col0 + 16 * j;
          if (full || (m < M && k < K))
            D[(16 * i + v) * K + 16 * j] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xffffu);
        }
  } else {
    float* D = static_cast<float*>(dX) + (m0 + row0) * K + k0 + col0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, k = k0 + col0 + 16 * j;
          if (full || (m < M && k < K)) D[(16 * i + v) * K + 16 * j] = acc[i][j][v];
        }
  }
}

}  // namespace

hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* AT2, int64_t Rp, void* dX, bool dx_bf16, hipStream_t st) {
  const int tm = (int)((M + TM - 1) / TM), tk = (int)((W.K + TK - 1) / TK);
  const unsigned grid = tile_grid(tm, tk);
  const int db = dx_bf16 ? 1 : 0;
  switch (2 * Rp / NSTEP) {
#define QNF4_DX_CASE(LS)                                                                      \
  case LS:                                                                                    \
    return timed_launch(kKernDxGemm, dx_gemm_kernel<LS>, dim3(grid), dim3(kThreads), st, W, dY, M, \
                        (const uint16_t*)sU, (const uint16_t*)AT2, Rp, dX, db, tm, tk, codebook());
    QNF4_DX_CASE(1)
    QNF4_DX_CASE(2)
    QNF4_DX_CASE(3)
    QNF4_DX_CASE(4)
    QNF4_DX_CASE(5)
    QNF4_DX_CASE(6)
    QNF4_DX_CASE(7)
    QNF4_DX_CASE(8)
#undef QNF4_DX_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qnf4
