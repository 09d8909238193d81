// Input gradient of the QLoRA linear layer, gfx950:
//   dX[M, K] = dY·Ŵ + s·U·A  =  [dY | sU_hi | sU_lo] · [Ŵ ; A ; A]
// (P1 简化版 and P2 §4.4: the gradient passes through the dequantized frozen
// weight; U = dY·B is the LoRA path's input gradient.)
//
// The reduction runs over the weight's rows n while the codes are contiguous
// along k, so the dequantized weight has to be transposed on its way to the
// MFMA B operand.  Design:
//   * 256x256 output tile per workgroup (token rows x input features), 4
//     waves; wave w owns the 64 output columns [64w, 64w+64), which lie in one
//     NF4 block per weight row.
//   * dY tiles (256 rows x 64 n) stream into double-buffered LDS by
//     buffer-to-LDS copies, as X does in the forward product.
//   * Per reduction step each wave dequantizes its 64 n x 64 k weight tile:
//       - lane i builds the 16-entry bf16 table RNE_bf16(fl32(q_j * c')) of
//         weight row i (the block's scaled codebook) in LDS;
//       - lane (rg, cg) owns rows 8rg..8rg+7 by columns 8cg..8cg+7; every
//         code becomes one 2-byte table read (two VALU ops for the address),
//         consecutive rows are paired in one register, so the values come
//         out already transposed (pairs along n) and go to a per-wave [k][n]
//         LDS tile;
//       - the wave reads its B fragments back from that tile.
//     Rows past N get an all-zero table, so a ragged last step adds nothing.
//   * The LoRA term is 2*Rp/64 extra steps with A = [sU_hi | sU_lo] and B read
//     from AT2[k][j] = A[j mod Rp][k] (a transposed, padded copy of A).
#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TK = 256, NSTEP = 64;

__device__ __forceinline__ int swz128(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}
// [k][n] weight tile: the chunk is XORed with (row ^ row/8) & 7 so that both
// the transposing writes (8 lanes per chunk column, rows 8 apart) and the
// fragment reads (16 consecutive rows) spread over all banks.
__device__ __forceinline__ int wswz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

template <int LSTEPS>
__global__ __launch_bounds__(256, 1) void dx_gemm_kernel(Nf4View W, const uint16_t* __restrict__ dY,
                                                         int64_t M, const uint16_t* __restrict__ sU,
                                                         const uint16_t* __restrict__ AT2,
                                                         int64_t Rp, void* __restrict__ dX,
                                                         int dx_bf16, int tiles_m, int tiles_k,
                                                         Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sa[2][TM * 128];   // dY tiles
  __shared__ __attribute__((aligned(16))) char swt[4][64 * 128];  // per-wave [k][n] weight tile
  // per-wave tables, 64 rows of 32 bytes; 256-byte alignment lets the
  // compiler OR (not add) a table offset into a table base
  __shared__ __attribute__((aligned(256))) char slut[4][64 * 32];
  __shared__ float sq[16];
  int tmi, tki;
  if (!tile_of(blockIdx.x, tiles_m, tiles_k, tmi, tki)) return;
  if (threadIdx.x < 16) sq[threadIdx.x] = cb.q[threadIdx.x];
  __syncthreads();

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int rg = lane >> 3, cg = lane & 7;
  const int64_t K = W.K, N = W.N;
  const int64_t m0 = (int64_t)tmi * TM;
  const int64_t kw0 = (int64_t)tki * TK + 64 * wave;  // first output column of this wave
  const int nsteps = (int)((N + NSTEP - 1) / NSTEP);
  const uint32_t kpr = (uint32_t)(K / kBlock);
  const uint32_t kbw = (uint32_t)(kw0 / kBlock);  // the wave's block column
  const bool wave_cols_ok = kw0 < K;
  const float mu = *W.mu;

  const rsrc_t rdy = make_rsrc(dY + m0 * N, (M - m0) * N * 2);
  const rsrc_t rsu = make_rsrc(sU + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t rc = make_rsrc(W.codes, N * (K / 2));
  const rsrc_t re = make_rsrc(W.e, N * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rat = make_rsrc(AT2 + kw0 * 2 * Rp, (K - kw0) * 2 * Rp * 2);

  // ---- dY (or sU) tile copies: wave w fills tile rows [64w, 64w+64)
  const int lrow = 64 * wave + (lane >> 3);
  const int lch = (lane & 7) ^ ((lane >> 3) & 7);
  const uint32_t vdy = (uint32_t)((lrow * N + 8 * lch) * 2);
  const uint32_t vsu = (uint32_t)((lrow * 2 * Rp + 8 * lch) * 2);
  const uint32_t dy_gstride = (uint32_t)(8 * N * 2), su_gstride = (uint32_t)(8 * 2 * Rp * 2);
  auto copy_dy = [&](char* t, int s) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(rdy, t + (64 * wave + 8 * c) * 128, vdy, c * dy_gstride + (uint32_t)s * 128u);
  };
  auto copy_su = [&](char* t, int l) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(rsu, t + (64 * wave + 8 * c) * 128, vsu, c * su_gstride + (uint32_t)l * 128u);
  };

  // ---- weight codes of step s: rows s*64 + 8rg + i, columns kw0 + 8cg .. +7
  const uint32_t vcode = (uint32_t)(8 * rg * (K / 2) + (kw0 + 8 * cg) / 2);
  const uint32_t code_rstride = (uint32_t)(K / 2);
  const uint32_t code_sstride = (uint32_t)(NSTEP * (K / 2));
  uint32_t cw[8];
  uint32_t eraw;
  float sraw;
  auto load_codes = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) cw[i] = buf_load4(rc, vcode, (uint32_t)s * code_sstride + i * code_rstride);
    // this lane's table row: n = s*64 + lane, block column kbw
    const uint32_t blk = ((uint32_t)s * NSTEP + lane) * kpr + kbw;
    eraw = buf_load1(re, blk, 0u);
    sraw = __uint_as_float(buf_load4(rs, (blk / kDqBlock) * 4u, 0u));
  };

  char* lut = slut[wave];
  const uint32_t lut_addr = lds_offset(lut);
  char* wt = swt[wave];
  // Table of row t (= lane) at slot 8*(t & 7) + ((t ^ (t >> 3)) & 7): slot mod
  // 8 (the bank group of a 32-byte table) differs across 8 consecutive t (the
  // table writes) and across t = 8rg + i for fixed i (one lookup instruction).
  const int my_slot = 8 * (lane & 7) + ((lane ^ (lane >> 3)) & 7);
  // row 8rg + i sits at slot 8i + (i ^ rg): byte offset 256i + 32(i ^ rg)
  u32x4_t bf[2][4][2];
  // Dequantize step s (codes already in cw/eraw/sraw) into bf[1].
  auto dequant = [&](int s) {
    const bool row_ok = wave_cols_ok && ((int64_t)s * NSTEP + lane < N);
    const float cp = decode_constant(eraw, sraw, mu);
    u32x4_t t0, t1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      t0[p] = row_ok ? pack_bf16x2(__fmul_rn(sq[2 * p], cp), __fmul_rn(sq[2 * p + 1], cp)) : 0u;
      t1[p] = row_ok ? pack_bf16x2(__fmul_rn(sq[8 + 2 * p], cp), __fmul_rn(sq[9 + 2 * p], cp)) : 0u;
    }
    *reinterpret_cast<u32x4_t*>(lut + my_slot * 32) = t0;
    *reinterpret_cast<u32x4_t*>(lut + my_slot * 32 + 16) = t1;
    // look up 8 rows x 8 columns, pairing rows (2p, 2p+1) in one register;
    // one column at a time keeps few lookups in flight (register pressure)
    uint32_t tab[8];  // table of row 8rg + i: 32-byte aligned LDS address
#pragma unroll
    for (int i = 0; i < 8; ++i) tab[i] = lut_addr + 256u * i + 32u * (uint32_t)(i ^ rg);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4_t o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        u16x2_t v;
        v.x = lds_read_u16(tab[2 * p] | code_x2(cw[2 * p], 4 * c));
        v.y = lds_read_u16(tab[2 * p + 1] | code_x2(cw[2 * p + 1], 4 * c));
        o[p] = __builtin_bit_cast(uint32_t, v);
      }
      *reinterpret_cast<u32x4_t*>(wt + wswz(8 * cg + c, rg)) = o;
      if (c & 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        bf[1][j][ks] = *reinterpret_cast<const u32x4_t*>(wt + wswz(16 * j + lr, 2 * kq + ks));
  };
  // LoRA B fragments of tail step l: AT2[kw0 + 16j + lr][64l + 16kq + 8ks ..]
  const uint32_t vat = (uint32_t)((lr * 2 * Rp + 16 * kq) * 2);
  const uint32_t at_jstride = (uint32_t)(16 * 2 * Rp * 2);
  auto load_at = [&](u32x4_t (&b)[4][2], int l) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b[j][0] = buf_load16(rat, vat, j * at_jstride + (uint32_t)l * 128u);
      b[j][1] = buf_load16(rat, vat, j * at_jstride + (uint32_t)l * 128u + 16u);
    }
  };
  auto roll = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf[0][j][0] = bf[1][j][0];
      bf[0][j][1] = bf[1][j][1];
    }
  };

  f32x4_t acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto mfma_step = [&](const char* t, const u32x4_t (&b)[4][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(t + swz128(16 * i + lr, 2 * kq + ks));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(a, b[j][ks], acc[i][j]);
      }
    }
  };

  // prologue: step 0
  copy_dy(sa[0], 0);
  load_codes(0);
  dequant(0);
  roll();
  wait_vmem();
  __syncthreads();

  for (int s = 0; s + 1 < nsteps; ++s) {
    copy_dy(sa[(s + 1) & 1], s + 1);
    load_codes(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(sa[s & 1], bf[0]);
    __builtin_amdgcn_sched_barrier(0);
    dequant(s + 1);
    wait_vmem();
    __syncthreads();
    roll();
  }
  // last weight step, prefetching LoRA step 0; then the unrolled LoRA tail
  copy_su(sa[nsteps & 1], 0);
  load_at(bf[1], 0);
  mfma_step(sa[(nsteps - 1) & 1], bf[0]);
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int l = 0; l < LSTEPS; ++l) {
    const int s = nsteps + l;
    if (l + 1 < LSTEPS) {
      copy_su(sa[(s + 1) & 1], l + 1);
      load_at(bf[l & 1], l + 1);
    }
    mfma_step(sa[s & 1], bf[(l + 1) & 1]);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane holds rows 16i + 4*kq + v of column kw0 + 16j + lr
  int row0 = 4 * kq, col0 = lr;
  asm volatile("" : "+v"(row0), "+v"(col0));
  const bool full = (m0 + TM <= M) && (kw0 + 64 <= K);
  if (dx_bf16) {
    uint16_t* D = static_cast<uint16_t*>(dX) + (m0 + row0) * K + kw0 + col0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, k = kw0 + col0 + 16 * j;
          if (full || (m < M && k < K))
            D[(16 * i + v) * K + 16 * j] = (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xffffu);
        }
  } else {
    float* D = static_cast<float*>(dX) + (m0 + row0) * K + kw0 + col0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + row0 + 16 * i + v, k = kw0 + col0 + 16 * j;
          if (full || (m < M && k < K)) D[(16 * i + v) * K + 16 * j] = acc[i][j][v];
        }
  }
}

// AT2[k][j] = A[j mod Rp][k] for (j mod Rp) < r, else 0;  [K, 2Rp] bf16.
__global__ void transpose_lora_a_kernel(const uint16_t* __restrict__ A, int64_t K, int r, int64_t Rp,
                                        uint16_t* __restrict__ AT2) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= K * 2 * Rp) return;
  const int64_t k = idx / (2 * Rp), j = (idx % (2 * Rp)) % Rp;
  AT2[idx] = j < r ? A[j * K + k] : (uint16_t)0;
}

}  // namespace

hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* A, int32_t r, int64_t Rp, uint16_t* AT2, void* dX,
                          bool dx_bf16, hipStream_t st) {
  const int64_t n2 = W.K * 2 * Rp;
  transpose_lora_a_kernel<<<(unsigned)((n2 + 255) / 256), 256, 0, st>>>(A, W.K, r, Rp, AT2);
  const int tm = (int)((M + TM - 1) / TM), tk = (int)((W.K + TK - 1) / TK);
  const unsigned grid = tile_grid(tm, tk);
  const int db = dx_bf16 ? 1 : 0;
  TimedLaunch tl(kKernDxGemm, st);
  switch (2 * Rp / NSTEP) {
#define QNF4_DX_CASE(LS) \
  case LS:               \
    dx_gemm_kernel<LS><<<grid, 256, 0, st>>>(W, dY, M, sU, AT2, Rp, dX, db, tm, tk, codebook()); \
    break;
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
