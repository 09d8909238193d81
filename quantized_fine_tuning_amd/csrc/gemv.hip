// Dequant-GEMV forward for few tokens (M <= 16), gfx950.
//
// P2 §六 and P5 (follow-up 1): at inference the 4-bit weight is dequantized to
// 16 bit on the fly for every product; with few tokens the product is bound by
// streaming the packed codes from HBM, so this path reads each code exactly
// once, keeps as many bytes in flight as possible and everything else small.
//
//   lora_down_small_kernel  T = X·Aᵀ (M x r, fp32) for one 16-wide slice of r
//                           per workgroup: 16 waves split K, all loads issued
//                           first, MFMA products, fixed-order combination of
//                           the 16 partial tiles.
//   gemv_kernel             one workgroup of 16 waves per 16 weight rows.  Lane
//                           (row l % 16, q = l / 16) owns whole NF4 blocks (64
//                           codes, one decoded constant c'); a "block group" is
//                           4 consecutive blocks of the 16 rows, q taking one
//                           each, and feeds 8 v_mfma_f32_16x16x32_bf16: MFMA t
//                           takes codes 8t..8t+7 of every lane's block (the
//                           A operand, X padded to 16 rows, uses the same
//                           k slots).  Wave w takes block groups w, w+16, ...;
//                           the codes, constants and X fragments of its next
//                           group are loaded before the current one is
//                           dequantized.  Each value is RNE_bf16(fl32(q_c * c'))
//                           with q_c read from a 16-entry LDS codebook (one
//                           address per code: no bank conflicts).  The LoRA
//                           term s·T·Bᵀ is 2 MFMAs per 32 ranks in wave 0 (A
//                           operand the bf16 hi/lo split of s·T), and the 16
//                           partial tiles are combined in a fixed order, one
//                           thread per output.
#include "host.h"

namespace qnf4 {
namespace {

constexpr int kWaves = 16, kThreads = 64 * kWaves;
constexpr int kDownSteps = 8;  // 32-wide K steps per wave and pass

// T = X·Aᵀ (M x r, fp32) for one 16-wide slice of r per workgroup of 16
// waves.  Wave w takes the 32-wide K steps w, w + 16, ...; each pass issues
// the loads of 8 steps before their MFMAs (for K = 4096 one pass: every load
// of the kernel is in flight at once).  The 16 partial tiles are combined in
// a fixed order.
template <bool F16>
__global__ __launch_bounds__(kThreads) void lora_down_small_kernel(const uint16_t* __restrict__ X,
                                                                   int M, int64_t K,
                                                                   const uint16_t* __restrict__ A,
                                                                   int r, float* __restrict__ T) {
  __shared__ f32x4_t s_acc[kWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int j0 = 16 * blockIdx.x;
  // A operand: X rows (tokens), B operand: rows of A (rank index); rows past
  // M or r read as zero
  const rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const rsrc_t ra = make_rsrc(A + (int64_t)j0 * K, (int64_t)(r - j0) * K * 2);
  const uint32_t vx = (uint32_t)((lr * K + 8 * kq) * 2);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // lane slot kq of step st holds k = 32st + 8kq .. +7
  const int64_t nst = K / 32;
  for (int64_t st0 = wave; st0 < nst; st0 += (int64_t)kWaves * kDownSteps) {
    u32x4_t xa[kDownSteps], ab[kDownSteps];
#pragma unroll
    for (int u = 0; u < kDownSteps; ++u) {
      const int64_t st = st0 + (int64_t)kWaves * u;
      const uint32_t off = st < nst ? (uint32_t)(st * 64) : 0x7fffffffu;  // past the end: zero
      xa[u] = buf_load16(rx, vx, off);
      ab[u] = buf_load16(ra, vx, off);
    }
#pragma unroll
    for (int u = 0; u < kDownSteps; ++u) acc = mfma16<F16>(xa[u], ab[u], acc);
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    // lane holds D rows (tokens) 4*(lane/16)+v of column (rank index) lane%16
    f32x4_t t = s_acc[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const f32x4_t a = s_acc[w][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) t[v] = __fadd_rn(t[v], a[v]);
    }
    const int j = j0 + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * (lane >> 4) + v;
      if (m < M && j < r) T[(int64_t)m * r + j] = t[v];
    }
  }
}

constexpr int GEMV_ROWS = 16;
constexpr int kGemvWaves = 16, kGemvThreads = 64 * kGemvWaves;

template <bool F16>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                            int M, const float* __restrict__ T,
                                                            const uint16_t* __restrict__ B, int r,
                                                            float scale, void* __restrict__ Y,
                                                            int y_bf16, Codebook cb) {
  __shared__ float sq[16];
  __shared__ f32x4_t s_acc[kGemvWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t K = W.K, N = W.N;
  const int64_t n0 = (int64_t)blockIdx.x * GEMV_ROWS;
  const int64_t nb = K / kBlock;         // blocks per row
  const int64_t ngroups = (nb + 3) / 4;  // block groups per row
  const uint32_t kpr = (uint32_t)nb;
  const float mu = *W.mu;
  // rows past N and blocks past the row read as zero (code 0 with c' = 0
  // would give 0; their products only reach unstored outputs or are zero)
  const rsrc_t rc = make_rsrc(W.codes + n0 * (K / 2), (N - n0) * (K / 2));
  const rsrc_t re = make_rsrc(W.e + n0 * kpr, (N - n0) * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const bool x_row = lr < M;

  struct Group {
    u32x4_t c[2];  // the lane's 64 codes
    uint32_t e;    // e4m3 byte
    float s;       // group scale
    u32x4_t x[8];  // X fragments of the 8 MFMAs (zero if lr >= M)
  };
  auto load = [&](Group& g, int64_t grp) __attribute__((always_inline)) {
    const int64_t b = 4 * grp + kq;  // this lane's block in its row
    const bool ok = grp < ngroups && b < nb;
    const uint32_t cb_off = ok ? (uint32_t)(lr * (K / 2) + b * 32) : 0x7fffffffu;
    g.c[0] = buf_load16(rc, cb_off, 0u);
    g.c[1] = buf_load16(rc, cb_off, 16u);
    const uint32_t blk = (uint32_t)(lr * kpr + b);
    g.e = buf_load1(re, ok ? blk : 0x7fffffffu, 0u);
    g.s = __uint_as_float(buf_load4(rs, ok ? (((uint32_t)n0 * kpr + blk) / kDqBlock) * 4u : 0x7fffffffu, 0u));
    // only the M token rows load X (the other lanes' A rows are zero)
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
    const float cp = decode_constant(g.e, g.s, mu);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t w = g.c[t >> 2][t & 3];  // codes 8t .. 8t+7
      u32x4_t bfrag;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        bfrag[p] = pack16<F16>(__fmul_rn(sq[(w >> (8 * p)) & 15u], cp),
                               __fmul_rn(sq[(w >> (8 * p + 4)) & 15u], cp));
      acc = mfma16<F16>(g.x[t], bfrag, acc);
    }
  };

  // The LoRA term s·T·Bᵀ enters wave 0's accumulator as extra MFMAs over
  // the rank in steps of 32: A operand the bf16 hi/lo split of s·T (token
  // row lr), B operand the workgroup's B rows (weight row lr); ranks past r
  // and tokens past M read as zero.
  const rsrc_t rt = make_rsrc(T, (int64_t)M * r * 4);
  const rsrc_t rb = make_rsrc(B + n0 * r, (N - n0) * r * 2);
  struct Lora {
    float t[8];
    uint32_t b[8];
  };
  auto lora_load = [&](Lora& l, int js) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 32 * js + 8 * kq + e;
      l.t[e] = __uint_as_float(buf_load4(rt, (x_row && j < r) ? (uint32_t)((lr * r + j) * 4) : 0x7fffffffu, 0u));
      l.b[e] = buf_load2(rb, j < r ? (uint32_t)((lr * r + j) * 2) : 0x7fffffffu, 0u);
    }
  };
  auto lora_mfma = [&](const Lora& l) __attribute__((always_inline)) {
    u32x4_t hi, lo, bf;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint16_t h0, l0, h1, l1;
      split_hilo16<F16>(__fmul_rn(scale, l.t[2 * p]), h0, l0);
      split_hilo16<F16>(__fmul_rn(scale, l.t[2 * p + 1]), h1, l1);
      hi[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      bf[p] = (l.b[2 * p] & 0xffffu) | (l.b[2 * p + 1] << 16);
    }
    acc = mfma16<F16>(hi, bf, acc);
    acc = mfma16<F16>(lo, bf, acc);
  };
  const int rsteps = (r + 31) / 32;

  // Everything this workgroup reads from memory is requested up front: the
  // first block group of every wave and, in wave 0, the LoRA operands, whose
  // MFMAs wave 0 issues before its main loop (their registers are free again
  // by then).
  Group ga, gb;
  load(ga, wave);
  if (wave == 0) {
    for (int js = 0; js < rsteps; js += 2) {
      Lora la[2];
      lora_load(la[0], js);
      if (js + 1 < rsteps) lora_load(la[1], js + 1);
      lora_mfma(la[0]);
      if (js + 1 < rsteps) lora_mfma(la[1]);
    }
  }
  if (tid < 16) sq[tid] = cb.q[tid];
  __syncthreads();  // codebook

  // two groups per iteration, alternating buffers: the loads of the next
  // group are issued (and kept above the barrier to the scheduler) before
  // the current group is consumed, and no loaded register is copied
  for (int64_t grp = wave; grp < ngroups; grp += 2 * kGemvWaves) {
    load(gb, grp + kGemvWaves);
    __builtin_amdgcn_sched_barrier(0);
    consume(ga);
    if (grp + kGemvWaves >= ngroups) break;
    load(ga, grp + 2 * kGemvWaves);
    __builtin_amdgcn_sched_barrier(0);
    consume(gb);
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  // one thread per output (token m, weight row n0 + c): the 16 partial tiles
  // in a fixed order
  if (tid < 16 * GEMV_ROWS) {
    const int m = tid >> 4, c = tid & 15;
    const int64_t nn = n0 + c;
    if (m < M && nn < N) {
      // partial tile of wave w: lane 16(m/4) + c holds token m in component m%4
      float y = s_acc[0][16 * (m >> 2) + c][m & 3];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) y = __fadd_rn(y, s_acc[w][16 * (m >> 2) + c][m & 3]);
      if (y_bf16)
        static_cast<uint16_t*>(Y)[(int64_t)m * N + nn] = (uint16_t)(pack16<F16>(y, 0.0f) & 0xffffu);
      else
        static_cast<float*>(Y)[(int64_t)m * N + nn] = y;
    }
  }
}

}  // namespace

hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float scale, void* Y, bool y16, float* T,
                       bool f16, hipStream_t st) {
  const unsigned gd = (unsigned)((r + 15) / 16);
  if (f16)
    lora_down_small_kernel<true><<<gd, kThreads, 0, st>>>(X, (int)M, W.K, A, r, T);
  else
    lora_down_small_kernel<false><<<gd, kThreads, 0, st>>>(X, (int)M, W.K, A, r, T);
  const unsigned grid = (unsigned)((W.N + GEMV_ROWS - 1) / GEMV_ROWS);
  return f16 ? timed_launch(kKernGemv, gemv_kernel<true>, dim3(grid), dim3(kGemvThreads), st, W, X, (int)M,
                            (const float*)T, B, r, scale, Y, y16 ? 1 : 0, codebook())
             : timed_launch(kKernGemv, gemv_kernel<false>, dim3(grid), dim3(kGemvThreads), st, W, X, (int)M,
                            (const float*)T, B, r, scale, Y, y16 ? 1 : 0, codebook());
}

}  // namespace qnf4
