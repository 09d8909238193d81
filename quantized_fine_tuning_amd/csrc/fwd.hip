// Forward product of the QLoRA linear layer for M > 16 tokens, gfx950:
//   Y[M, N] = X·Ŵᵀ + s·T·Bᵀ  =  [X | sT_hi | sT_lo] · [Ŵ | B | B]ᵀ
// (P1 §七 dataflow figure: the 4-bit base is dequantized to BF16 for the
// matmul and the LoRA path is added to the output.)
//
// Design
//   * 256x256 output tile per workgroup, 4 waves; wave w owns the 64 weight
//     rows [64w, 64w+64) of the tile and all 256 token rows, so every weight
//     element is dequantized exactly once per workgroup, straight into
//     registers: each lane turns 8 bytes of codes (16 consecutive k of one
//     weight row) into the bf16 B operand of two v_mfma_f32_16x16x32_bf16.
//     Within a 64-wide reduction step lane group q = lane/16 holds k in
//     [16q, 16q+16); the A operand (X from LDS) uses the same k slots.
//   * Dequantization goes through a per-row table: per step lane t writes
//     the 16 values RNE_bf16(fl32(q_j * c')) of weight row 64w + t to LDS, and
//     each code then costs one 2-byte table read (bit-identical to
//     multiplying per element, since the value depends only on code and row).
//   * X goes through a double-buffered LDS tile (256 rows x 64 k, 16-byte
//     chunks XOR-swizzled by row) filled by buffer-to-LDS copies one step
//     ahead (no staging registers); the codes of the next step are loaded one
//     step ahead and dequantized after the current step's MFMAs are issued.
//   * All operand reads are buffer loads whose resources end at the tensor's
//     last row, so ragged tiles read zeros without per-lane branches.
//   * The LoRA up-projection is 2*Rp/64 extra reduction steps whose A operand
//     is the bf16 hi/lo split of s·T and whose B operand is the padded copy
//     B2 = [B | 0 | B | 0] ([N, 2Rp] bf16).
//   * Workgroups are mapped to tiles so that each XCD (workgroup id mod 8)
//     walks a contiguous run of a grouped tile order (4 M-tiles per group):
//     the ~32 workgroups resident on one XCD share X and code rows in its L2.
#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TN = 256, KSTEP = 64;

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int LSTEPS>
__global__ __launch_bounds__(256, 1) void fwd_gemm_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                          int64_t M, const uint16_t* __restrict__ sT,
                                                          const uint16_t* __restrict__ B2,
                                                          int64_t Rp, void* __restrict__ Y,
                                                          int y_bf16, int tiles_m, int tiles_n,
                                                          Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sx[2][TM * 128];
  // per-wave tables: 64 weight rows x 16 bf16 (32 bytes); 256-byte alignment
  // lets the compiler OR a table offset into a table base
  __shared__ __attribute__((aligned(256))) char slut[4][64 * 32];
  __shared__ float sq[16];
  int tmi, tni;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, tmi, tni)) return;
  if (threadIdx.x < 16) sq[threadIdx.x] = cb.q[threadIdx.x];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
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

  // X tile: wave w copies tile rows [64w, 64w+64) straight into LDS, 8 rows
  // (1 KB) per instruction.  Lane i lands in physical chunk i & 7 of row
  // (i >> 3) of the group, so it fetches logical chunk (i & 7) ^ (i >> 3),
  // which keeps the XOR swizzle of xswz().
  const int lrow = 64 * wave + (lane >> 3);
  const int lch = (lane & 7) ^ ((lane >> 3) & 7);
  const uint32_t vx = (uint32_t)((lrow * K + 8 * lch) * 2);
  const uint32_t vt = (uint32_t)((lrow * 2 * Rp + 8 * lch) * 2);
  const uint32_t x_gstride = (uint32_t)(8 * K * 2), t_gstride = (uint32_t)(8 * 2 * Rp * 2);
  auto copy_x = [&](char* t, int s) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(rx, t + (64 * wave + 8 * c) * 128, vx, c * x_gstride + (uint32_t)s * 128u);
  };
  auto copy_t = [&](char* t, int l) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(rt, t + (64 * wave + 8 * c) * 128, vt, c * t_gstride + (uint32_t)l * 128u);
  };

  // B operand: this lane's weight rows are 64*wave + 16j + lr (tile-local)
  const int brow = 64 * wave + lr;
  const uint32_t vc = (uint32_t)(brow * (K / 2) + 8 * kq);
  const uint32_t vb = (uint32_t)((brow * 2 * Rp + 16 * kq) * 2);
  const uint32_t c_rstride = (uint32_t)(16 * (K / 2));
  const uint32_t b_rstride = (uint32_t)(16 * 2 * Rp * 2);
  u32x2_t craw[4];
  uint32_t eraw;
  float sraw;
  // codes of rows 16j + lr (16 consecutive k each); the e4m3 byte and group
  // scale of this lane's table row 64*wave + lane
  const uint32_t ve_me = (uint32_t)(64 * wave + lane) * kpr;
  const uint32_t blk_me = (uint32_t)(n0 + 64 * wave + lane) * kpr;
  auto load_codes = [&](int s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) craw[j] = buf_load8(rc, vc, j * c_rstride + (uint32_t)s * 32u);
    eraw = buf_load1(re, ve_me, (uint32_t)s);
    sraw = __uint_as_float(buf_load4(rs, ((blk_me + (uint32_t)s) / kDqBlock) * 4u, 0u));
  };
  // B fragments of two consecutive steps (ping-pong, no copies)
  u32x4_t bf[2][4][2];
  char* lut = slut[wave];
  const uint32_t lut_base = lds_offset(lut) + (uint32_t)lr * 32u;  // row 16j + lr adds 512j
  // Dequantize: lane t writes the table RNE_bf16(fl32(q_j * c')) of row t,
  // then every code is one 2-byte lookup in the table of its row; pairs of
  // consecutive k share a register.  (Rows past N only feed output columns
  // past N, which are not stored.)
  auto make_b = [&](u32x4_t (&b)[4][2]) {
    const float cp = decode_constant(eraw, sraw, mu);
    u32x4_t t0, t1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      t0[p] = pack_bf16x2(__fmul_rn(sq[2 * p], cp), __fmul_rn(sq[2 * p + 1], cp));
      t1[p] = pack_bf16x2(__fmul_rn(sq[8 + 2 * p], cp), __fmul_rn(sq[9 + 2 * p], cp));
    }
    *reinterpret_cast<u32x4_t*>(lut + lane * 32) = t0;
    *reinterpret_cast<u32x4_t*>(lut + lane * 32 + 16) = t1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t tab = lut_base + (uint32_t)(16 * j) * 32u;  // 32-byte aligned
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t w = craw[j][ks];
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          u16x2_t v;
          v.x = lds_read_u16(tab | code_x2(w, 8 * p));
          v.y = lds_read_u16(tab | code_x2(w, 8 * p + 4));
          o[p] = __builtin_bit_cast(uint32_t, v);
        }
        b[j][ks] = o;
      }
    }
  };
  auto load_b2 = [&](u32x4_t (&b)[4][2], int l) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b[j][0] = buf_load16(rb, vb, j * b_rstride + (uint32_t)l * 128u);
      b[j][1] = buf_load16(rb, vb, j * b_rstride + (uint32_t)l * 128u + 16u);
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
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(t + xswz(16 * i + lr, 2 * kq + ks));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32(a, b[j][ks], acc[i][j]);
      }
    }
  };

  auto roll = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf[0][j][0] = bf[1][j][0];
      bf[0][j][1] = bf[1][j][1];
    }
  };

  // prologue: step 0 (K >= 64, so step 0 is a weight step)
  copy_x(sx[0], 0);
  load_codes(0);
  __syncthreads();  // codebook in LDS
  make_b(bf[0]);
  wait_vmem();
  __syncthreads();

  // Weight steps 0 .. ksteps-2: prefetch step s+1 (X into the other LDS
  // buffer, codes into registers), MFMAs of step s, dequantize step s+1.
  // One step per iteration and no other loop carrying the accumulators:
  // anything else makes the register allocator shuffle or spill them.
  for (int s = 0; s + 1 < ksteps; ++s) {
    copy_x(sx[(s + 1) & 1], s + 1);
    load_codes(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(sx[s & 1], bf[0]);
    __builtin_amdgcn_sched_barrier(0);
    make_b(bf[1]);
    wait_vmem();
    __syncthreads();
    roll();
  }
  // Last weight step, prefetching LoRA step 0; then the LoRA steps, unrolled
  // (A = [sT_hi | sT_lo] from LDS, B = B2 fragments loaded into registers).
  copy_t(sx[ksteps & 1], 0);
  load_b2(bf[1], 0);
  mfma_step(sx[(ksteps - 1) & 1], bf[0]);
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int l = 0; l < LSTEPS; ++l) {
    const int s = ksteps + l;
    if (l + 1 < LSTEPS) {
      copy_t(sx[(s + 1) & 1], l + 1);
      load_b2(bf[l & 1], l + 1);
    }
    mfma_step(sx[s & 1], bf[(l + 1) & 1]);
    wait_vmem();
    __syncthreads();
  }

  // epilogue: lane holds rows 16i + 4*kq + v of column 64*wave + 16j + lr.
  // The row/column bases go through an empty asm so that their address
  // arithmetic is not hoisted above the main loop (it would stay live there).
  int row0 = 4 * kq, col0 = 64 * wave + lr;
  asm volatile("" : "+v"(row0), "+v"(col0));
  const bool full = (m0 + TM <= M) && (n0 + TN <= N);
  if (y_bf16) {
    uint16_t* Yb = static_cast<uint16_t*>(Y) + (m0 + row0) * N + n0 + col0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
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
    for (int i = 0; i < 16; ++i)
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
  TimedLaunch tl(kKernFwdGemm, st);
  switch (2 * Rp / KSTEP) {
#define QNF4_FWD_CASE(LS) \
  case LS:                \
    fwd_gemm_kernel<LS><<<grid, 256, 0, st>>>(W, X, M, sT, B2, Rp, Y, yb, tm, tn, codebook()); \
    break;
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
