// Dequant-GEMV forward for few tokens (M <= 16), gfx950.
//
// P2 §六 and P5 (follow-up 1): at inference the 4-bit weight is dequantized to
// 16 bit on the fly for every product; with few tokens the product is bound by
// streaming the packed codes from HBM, so this path reads each code exactly
// once, keeps as many bytes in flight as possible and everything else small.
// Two launches:
//
//   lora_down_split_kernel  partial products of T = X·Aᵀ: one workgroup of 4
//                           waves per slice of K (256 wide, wider above
//                           K = 4096 so that there are at most 16 slices:
//                           768 at K = 11008, where the down projection's
//                           forward at M = 4 went from 16.4 to 15.0 us) and
//                           16 ranks, MFMA products, the 4 waves' tiles
//                           summed in a fixed order; a tiny grid
//                           (K/slice x r/16 workgroups).
//   gemv_kernel             one workgroup per 16 weight rows: 16 waves, or,
//                           when the weight has more row groups than the
//                           chip has compute units, 8 waves if X fits 32 KB
//                           (two workgroups resident per unit, one streaming
//                           its codes while the other decodes: the 11008 x
//                           4096 gate forward at M = 4 went from 23.0 to
//                           17.8 us graph-replayed) and 4 waves if it fits
//                           8 KB (three per unit: all 688 row groups of the
//                           gate resident at once; M = 1 went from 17.6 us
//                           with 16 waves and 15.7 with 8 to 14.4).  Each
//                           wave sums its block groups in order before the
//                           fixed-order sum over waves.
//                           Lane (row l % 16, q = l / 16) owns whole NF4 blocks
//                           (64 codes, one decoded constant c'); a "block
//                           group" is 4 consecutive blocks of the 16 rows, q
//                           taking one each, and feeds 8
//                           v_mfma_f32_16x16x32_bf16: MFMA t takes codes
//                           8t..8t+7 of every lane's block (the A operand, X
//                           padded to 16 rows and staged in LDS up to 128 KB,
//                           uses the same k slots).  Each value is
//                           RNE_bf16(fl32(q_c * c')) with q_c read from a
//                           16-entry LDS codebook (one address per code: no
//                           bank conflicts).  The waves' partial tiles are
//                           combined in a fixed order, one thread per output,
//                           which also adds s·Σ_j T[m][j]·B[n][j] in fp32, T
//                           summed from the split kernel's partial tiles in
//                           slice order.
//
// Measured on the 4096x4096 q_proj weight (M = 1, graph-replayed forwards):
// computing T inside every workgroup (each reading all of A) delayed the data
// by ~3.4 us; summing the partial tiles with loads issued one after the other
// in the epilogue cost ~3.7 us; the X fragments loaded by every wave from
// global memory ~1.6 us.  The partial tiles, written by the launch just
// before, arrive late when requested at the kernel's start (the forward took
// 10.8 us with them first, 9.1 us with them requested right after the codes
// and summed in the epilogue; 8.0 us without them at all).  Nothing that the
// first barrier waits for is requested after the codes: loads complete in
// issue order, so such a wait would also wait for them.
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int GEMV_ROWS = 16;
constexpr int kTSlice = 256;  // reduction elements per T partial tile (the narrowest)
constexpr int kPre = 16;       // partial tiles a GEMV thread requests at its start
// Slice width for a reduction of K: 256, or a multiple of 256 that keeps
// the slice count within kPre (up to 1024, K <= 16384), so that every GEMV
// thread requests its partial tiles right after its codes.
inline int t_slice(int64_t K) {
  const int64_t u = (K + (int64_t)kTSlice * kPre - 1) / ((int64_t)kTSlice * kPre);
  return kTSlice * (int)(u < 1 ? 1 : (u > 4 ? 4 : u));
}

// Partial tiles of T = X·Aᵀ: workgroup (s, jt) sums k in [128·UC·s, +128·UC)
// for ranks [16jt, +16) and all 16 token rows (rows past M, ranks past r and
// k past K read as zero), 4 waves of 32·UC k each, and writes the 16 x 16
// tile P[(s * JT + jt) * 256 + 16m + j] (fp32).
template <bool F16, int UC>
__global__ __launch_bounds__(256) void lora_down_split_kernel(const uint16_t* __restrict__ X, int M, int64_t K,
                                                              const uint16_t* __restrict__ A, int r,
                                                              float* __restrict__ P) {
  __shared__ f32x4_t s_acc[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t slice = blockIdx.x, jt = blockIdx.y, JT = gridDim.y;
  const rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const int64_t j0 = 16 * jt;
  const rsrc_t ra = make_rsrc(A + j0 * K, ((int64_t)r - j0) * K * 2);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // slice of 128·UC reduction elements: wave w takes [32·UC·w, +32·UC)
  u32x4_t xa[UC], ab[UC];
#pragma unroll
  for (int u = 0; u < UC; ++u) {
    const int64_t k = slice * (128 * UC) + 32 * UC * wave + 32 * u + 8 * kq;
    const uint32_t off = k < K ? (uint32_t)((lr * K + k) * 2) : 0x7fffffffu;
    xa[u] = buf_load16(rx, off, 0u);
    ab[u] = buf_load16(ra, off, 0u);
  }
#pragma unroll
  for (int u = 0; u < UC; ++u) acc = mfma16<F16>(xa[u], ab[u], acc);
  s_acc[wave][lane] = acc;
  __syncthreads();
  // thread (m, j): lane 16(m/4) + j holds token m in component m%4
  const int m = tid >> 4, j = tid & 15;
  const int sl = 16 * (m >> 2) + j, v = m & 3;
  float t = s_acc[0][sl][v];
#pragma unroll
  for (int w = 1; w < 4; ++w) t = __fadd_rn(t, s_acc[w][sl][v]);
  P[(slice * JT + jt) * 256 + 16 * m + j] = t;
}

// The adapter term of the GEMV, T[m][j] = Σ_s P[s][m][j] summed in slice
// order into t_fin (stride 257 floats per token row); workgroup 0 also
// writes T_out.  With at most kPre slices and one entry per thread the
// thread's partials were requested at the start of the kernel (`pre`);
// otherwise gemv_t_reduce loads them, 16 at a time, all independent.
__device__ __forceinline__ void gemv_t_store(int r, int idx, float t, float* t_fin, float* __restrict__ T_out) {
  t_fin[(idx / r) * 257 + idx % r] = t;
  if (T_out && blockIdx.x == 0) T_out[idx] = t;
}
__device__ __forceinline__ void gemv_t_reduce(int nthreads, int M, int r, const float* __restrict__ P, int S,
                                              int JT, float* t_fin, float* __restrict__ T_out) {
  const int64_t sstride = (int64_t)JT * 256;
  for (int idx = threadIdx.x; idx < M * r; idx += nthreads) {
    const int m = idx / r, j = idx % r;
    const float* p = P + (int64_t)(j >> 4) * 256 + 16 * m + (j & 15);
    float t = 0.0f;
    for (int s0 = 0; s0 < S; s0 += kPre) {
      float v[kPre];
#pragma unroll
      for (int i = 0; i < kPre; ++i) v[i] = s0 + i < S ? p[(int64_t)(s0 + i) * sstride] : 0.0f;
#pragma unroll
      for (int i = 0; i < kPre; ++i)
        if (s0 + i < S) t = (s0 + i == 0) ? v[i] : __fadd_rn(t, v[i]);
    }
    gemv_t_store(r, idx, t, t_fin, T_out);
  }
}

constexpr int kGemvWaves = 16, kGemvThreads = 64 * kGemvWaves;  // the widest workgroup
constexpr int kGemvXLdsBytes = 128 * 1024;  // X staged in LDS up to this size
// The adapter term's t_fin [16][257] and s_b [16][256]: arrays of their own,
// except with X of more than 32 KB staged (up to 128 KB), where they take
// X's place after the main loop.
constexpr int kTfinFloats = 16 * 257, kSbFloats = 16 * 256;
constexpr size_t kGemvEpiBytes = (size_t)(kTfinFloats + kSbFloats) * 4;
// LDS of a workgroup (the device's 160 KB): s_acc (16 KB) and the codebook
// (256 bytes with its alignment) beside the X region; beside X of up to
// 32 KB also t_fin and s_b.
constexpr size_t kGemvAccBytes = (size_t)16 * 64 * 16 + 256;
static_assert(kGemvAccBytes + kGemvXLdsBytes <= 160 * 1024, "X staged up to 128 KB fits the LDS");
static_assert(kGemvAccBytes + 32 * 1024 + kGemvEpiBytes <= 160 * 1024, "X of 32 KB fits beside the epilogue arrays");

// WV waves per 16 weight rows; each wave's next block group is requested
// before the current one is dequantized.  XV > 0: X (M x K bf16) is staged
// in LDS once per workgroup, XV 16-byte pieces per thread (XV·WV KB: 32 KB
// for (2, 16) and (4, 8), 8 KB for (2, 4), 128 KB for (8, 16)), and the
// MFMA fragments are read from there; XV = 0:
// every wave loads its fragments from global memory (the same few bytes
// requested by every wave of every workgroup at once cost ~1.6 us at M = 1
// on the q_proj weight, ~2 us at M = 16, measured).
template <bool F16, int XV, int WV>
__global__ __launch_bounds__(64 * WV) void gemv_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                            int M, const float* __restrict__ P, int S, int JT,
                                                            const uint16_t* __restrict__ B, int r,
                                                            float scale, void* __restrict__ Y,
                                                            int y_bf16, float* __restrict__ T_out, Codebook cb) {
  constexpr int NW = WV, NT = 64 * WV;  // waves and threads of the workgroup
  static_assert(NT >= 16 * GEMV_ROWS, "one thread per output of a 16-token x 16-row tile");
  constexpr bool XL = XV > 0;  // X staged: XV 16-byte pieces per thread
  constexpr bool epi_late = XV * NT * 16 > 32 * 1024;  // t_fin and s_b in X's place
  extern __shared__ __attribute__((aligned(16))) char sx[];  // X [M][K] bf16 (XL)
  __shared__ float t_fin_own[epi_late ? 1 : kTfinFloats];
  __shared__ float s_b_own[epi_late ? 1 : kSbFloats];
  float* const t_fin = epi_late ? reinterpret_cast<float*>(sx) : t_fin_own;
  float* const s_b = epi_late ? reinterpret_cast<float*>(sx) + kTfinFloats : s_b_own;
  __shared__ __attribute__((aligned(256))) float sq[16];  // low address byte free for 4·code
  __shared__ f32x4_t s_acc[NW][64];
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
    if (!XL && x_row) {
      const uint32_t xo = ok ? (uint32_t)((lr * K + b * kBlock) * 2) : 0x7fffffffu;
#pragma unroll
      for (int t = 0; t < 8; ++t) g.x[t] = buf_load16(rx, xo, 16u * t);
    }
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Group& g, int64_t grp) __attribute__((always_inline)) {
    const float cp = decode_constant(g.e, g.s, mu);
    const int64_t b = 4 * grp + kq;
    const bool use_x = x_row && grp < ngroups && b < nb;
    const char* xrow = sx + (size_t)(lr * K + (use_x ? b : 0) * kBlock) * 2;
    // level of a code: one read of the fp32 codebook at sq + 4·code, the
    // address formed four codes at a time (byte j of we / wo is 4·code of
    // the even / odd code of byte j of w) and put in place by a byte permute
    const uint32_t sqb = lds_offset(sq);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t w = g.c[t >> 2][t & 3];  // codes 8t .. 8t+7
      const uint32_t we = (w << 2) & 0x3C3C3C3Cu, wo = (w >> 2) & 0x3C3C3C3Cu;
      u32x4_t bfrag;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float qe = *(const __attribute__((address_space(3))) float*)(uintptr_t)__builtin_amdgcn_perm(
            sqb, we, 0x07060500u | (uint32_t)p);
        const float qo = *(const __attribute__((address_space(3))) float*)(uintptr_t)__builtin_amdgcn_perm(
            sqb, wo, 0x07060500u | (uint32_t)p);
        bfrag[p] = pack16<F16>(__fmul_rn(qe, cp), __fmul_rn(qo, cp));
      }
      u32x4_t xa = g.x[t];
      if constexpr (XL) xa = use_x ? *reinterpret_cast<const u32x4_t*>(xrow + 16 * t) : u32x4_t{0u, 0u, 0u, 0u};
      acc = mfma16<F16>(xa, bfrag, acc);
    }
  };

  // Requested first, so that waiting for them does not wait for the codes
  // (loads complete in issue order): 8 values of the workgroup's B rows
  // (16·r contiguous bf16), and X when staged.
  const rsrc_t rbr = make_rsrc(B + n0 * r, (N - n0) * r * 2);
  const u32x4_t braw = buf_load16(rbr, tid < 2 * r ? (uint32_t)(16 * tid) : 0x7fffffffu, 0u);
  u32x4_t xs[XL ? XV : 1];
  if constexpr (XL) {
    const int nvec = (M * (int)K * 2) / 16;
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int v = tid + i * NT;
      xs[i] = buf_load16(rx, v < nvec ? (uint32_t)(16 * v) : 0x7fffffffu, 0u);
    }
  }
  // (the codebook is indexed per thread, so it is read from memory too)
  const float cbq = cb.q[tid & 15];
  __builtin_amdgcn_sched_barrier(0);
  Group ga, gb;
  load(ga, wave);
  __builtin_amdgcn_sched_barrier(0);
  // This thread's T entry (token tid / r, rank tid % r): its partial tiles,
  // written by the split kernel just before this launch, requested after
  // the codes (read at the start of the kernel, they took ~1.5 us longer to
  // arrive than the codes themselves) and summed in the epilogue.
  const bool t_pre = XL && S <= kPre && M * r <= NT;
  float pre[kPre];
  if (t_pre && wave * 64 < M * r) {
    const int tm = tid / r, tj = tid % r;
    const rsrc_t rp = make_rsrc(P, (int64_t)S * JT * 256 * 4);
    const uint32_t po = (uint32_t)(((tj >> 4) * 256 + 16 * tm + (tj & 15)) * 4);
    // (the whole offset in the lane's register: it alone is range-checked)
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      pre[i] = __uint_as_float(
          buf_load4(rp, tid < M * r && i < S ? po + (uint32_t)(i * JT * 256 * 4) : 0x7fffffffu, 0u));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XL) {
    const int nvec = (M * (int)K * 2) / 16;
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int v = tid + i * NT;
      if (v < nvec) *reinterpret_cast<u32x4_t*>(sx + 16 * v) = xs[i];
    }
  }
  if (tid < 16) sq[tid] = cbq;
  // the B rows widened to fp32 into s_b [16][r] (after the main loop when
  // s_b lies in X's place)
  auto stage_b = [&]() __attribute__((always_inline)) {
    if (tid < 2 * r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_b[8 * tid + 2 * i] = widen16<F16>(braw[i] & 0xffffu);
        s_b[8 * tid + 2 * i + 1] = widen16<F16>(braw[i] >> 16);
      }
    }
  };
  if (!epi_late) stage_b();
  __syncthreads();  // codebook, X, B rows

  // two groups per iteration, alternating buffers: the loads of the next
  // group are issued (and kept above the barrier to the scheduler) before
  // the current group is consumed, and no loaded register is copied
  for (int64_t grp = wave; grp < ngroups; grp += 2 * NW) {
    load(gb, grp + NW);
    __builtin_amdgcn_sched_barrier(0);
    consume(ga, grp);
    if (grp + NW >= ngroups) break;
    load(ga, grp + 2 * NW);
    __builtin_amdgcn_sched_barrier(0);
    consume(gb, grp + NW);
  }
  s_acc[wave][lane] = acc;
  if (epi_late) {
    __syncthreads();  // X read by every wave: its region takes t_fin and s_b
    stage_b();
  }
  if (t_pre) {
    if (tid < M * r) {
      float t = pre[0];
#pragma unroll
      for (int i = 1; i < kPre; ++i)
        if (i < S) t = __fadd_rn(t, pre[i]);
      gemv_t_store(r, tid, t, t_fin, T_out);
    }
  } else {
    gemv_t_reduce(NT, M, r, P, S, JT, t_fin, T_out);
  }
  __syncthreads();
  // one thread per output (token m, weight row n0 + c): the 16 partial
  // tiles in a fixed order, then the adapter term
  // fl32(s · Σ_j T[m][j]·B[n0 + c][j]) in fp32, j in order
  if (tid < 16 * GEMV_ROWS) {
    const int m = tid >> 4, c = tid & 15;
    const int64_t nn = n0 + c;
    if (m < M && nn < N) {
      float y = s_acc[0][16 * (m >> 2) + c][m & 3];
#pragma unroll
      for (int w = 1; w < NW; ++w) y = __fadd_rn(y, s_acc[w][16 * (m >> 2) + c][m & 3]);
      float dot = 0.0f;
      for (int j = 0; j < r; ++j) dot = __fadd_rn(dot, __fmul_rn(t_fin[m * 257 + j], s_b[c * r + j]));
      y = __fadd_rn(y, __fmul_rn(scale, dot));
      if (y_bf16)
        static_cast<uint16_t*>(Y)[(int64_t)m * N + nn] = (uint16_t)(pack16<F16>(y, 0.0f) & 0xffffu);
      else
        static_cast<float*>(Y)[(int64_t)m * N + nn] = y;
    }
  }
}

}  // namespace

size_t gemv_partial_bytes(int64_t K, int32_t r) {
  const int sl = t_slice(K);
  return (size_t)((K + sl - 1) / sl) * (size_t)((r + 15) / 16) * 256 * 4;
}

hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                       int32_t r, float scale, void* Y, bool y16, float* T, float* P, bool f16, hipStream_t st) {
  const int sl = t_slice(W.K);
  const int S = (int)((W.K + sl - 1) / sl), JT = (r + 15) / 16;
  const dim3 tg((unsigned)S, (unsigned)JT);
  // 128·UC reduction elements per slice: UC = 2, 4, 6 or 8
#define QNF4_SPLIT_LAUNCH(UC)                                                                  \
  if (f16)                                                                                     \
    lora_down_split_kernel<true, UC><<<tg, 256, 0, st>>>(X, (int)M, W.K, A, r, P);             \
  else                                                                                         \
    lora_down_split_kernel<false, UC><<<tg, 256, 0, st>>>(X, (int)M, W.K, A, r, P);
  switch (sl / 128) {
    case 2: QNF4_SPLIT_LAUNCH(2) break;
    case 4: QNF4_SPLIT_LAUNCH(4) break;
    case 6: QNF4_SPLIT_LAUNCH(6) break;
    default: QNF4_SPLIT_LAUNCH(8) break;
  }
#undef QNF4_SPLIT_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((W.N + GEMV_ROWS - 1) / GEMV_ROWS);
  const int yb = y16 ? 1 : 0;
  const size_t xb = (size_t)M * W.K * 2;
  const bool xl = xb <= (size_t)kGemvXLdsBytes;
  const bool x2 = xb <= 32 * 1024;
  const size_t shm = x2 ? xb : (xl ? std::max(xb, kGemvEpiBytes) : 0);
  // More row groups than compute units: workgroups of 8 waves (two resident
  // per compute unit, so that the next workgroup's codes stream while one
  // decodes), or of 4 with X within 8 KB (three resident: every row group
  // of a 688-group weight at once) and r <= 128 (the workgroup's 16 B rows
  // are staged 16 bytes a thread); otherwise 16 waves, one workgroup per
  // unit.
  const bool narrow = grid > 256 && xb <= 32 * 1024;
  const bool four = narrow && xb <= 8 * 1024 && 2 * r <= 64 * 4;
#define QNF4_GEMV_LAUNCH(XV, WV)                                                                                \
  return f16 ? timed_launch_shm(kKernGemv, gemv_kernel<true, XV, WV>, dim3(grid), dim3(64 * WV), shm, st, W, X, \
                                (int)M, (const float*)P, S, JT, B, r, scale, Y, yb, T, codebook())      \
             : timed_launch_shm(kKernGemv, gemv_kernel<false, XV, WV>, dim3(grid), dim3(64 * WV), shm, st, W, X, \
                                (int)M, (const float*)P, S, JT, B, r, scale, Y, yb, T, codebook())
  // X staged with 2 or 8 pieces of 16 bytes per thread (up to 32 or 128 KB)
  if (four) QNF4_GEMV_LAUNCH(2, 4);
  if (narrow) QNF4_GEMV_LAUNCH(4, 8);
  if (x2) QNF4_GEMV_LAUNCH(2, 16);
  if (xl) QNF4_GEMV_LAUNCH(8, 16);
  QNF4_GEMV_LAUNCH(0, 16);
#undef QNF4_GEMV_LAUNCH
}

}  // namespace qnf4
