// Low-rank side products of the QLoRA linear layer for gfx950.
//
// P1 §七 (dataflow figure): the frozen 4-bit weight is dequantized to BF16 and
// multiplied with the BF16 activation, and the trainable LoRA path is added to
// the output.  P1 简化版 and P2 §4.4: the backward pass sends the gradient
// through the dequantized frozen weight into LoRA A and B only.
//
// All products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Every
// kernel here is an instance of one tile engine:
//   * operands are staged per 64-wide reduction step in LDS as bf16 tiles whose
//     rows are contiguous along the reduction (128 bytes per row, 16-byte chunks
//     XOR-swizzled by row to keep fragment reads free of bank conflicts),
//     double buffered, one barrier per step;
//   * "loaders" fill a tile from global memory: plain bf16 rows, or bf16 read
//     across rows (transposed on the way into LDS).
// The kernels here are the low-rank side products (T = X·Aᵀ, U = dY·B, and the
// split-M reductions of dA and dB); the two big dequantizing products live in
// fwd.hip and dx.hip.  Their LoRA terms are extra reduction steps over
// [s·T_hi | s·T_lo] and [s·U_hi | s·U_lo] (bf16 hi/lo splits of the fp32
// intermediates, so the low-rank path keeps ~16 significant bits), which the
// kernels here produce.
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int KS = 64;          // reduction elements per step
constexpr int ROW_BYTES = 128;  // one tile row: 64 bf16

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ (row & 7)) << 4);
}

// ---------------------------------------------------------------------------
// Tile engine
// ---------------------------------------------------------------------------

template <int MT, int NT, int WM, int WN>
struct Core {
  static constexpr int FM = MT / WM / 16;
  static constexpr int FN = NT / WN / 16;
  f32x4_t acc[FM][FN];

  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  __device__ void step(const char* sA, const char* sB, int wm, int wn, int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(sA + swz((wm * FM + i) * 16 + r, ks * 4 + q));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(sB + swz((wn * FN + j) * 16 + r, ks * 4 + q));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
    }
  }
};

// Runs the reduction; `LA` fills the A tile (MT rows), `LB` the B tile (NT rows).
template <int MT, int NT, int WM, int WN, class LA, class LB>
__device__ __forceinline__ void run_tiles(Core<MT, NT, WM, WN>& core, LA& la, LB& lb, int nsteps,
                                          char* smem) {
  constexpr int A_BYTES = MT * ROW_BYTES, B_BYTES = NT * ROW_BYTES;
  char* sA[2] = {smem, smem + A_BYTES + B_BYTES};
  char* sB[2] = {smem + A_BYTES, smem + 2 * A_BYTES + B_BYTES};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  core.zero();
  if (nsteps <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(sA[0]);
  lb.store(sB[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      la.load(s + 1);
      lb.load(s + 1);
    }
    core.step(sA[cur], sB[cur], wm, wn, lane);
    if (more) {
      la.store(sA[cur ^ 1]);
      lb.store(sB[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Visit every accumulator element: f(row, col, value), rows/cols tile-local.
template <int MT, int NT, int WM, int WN, class F>
__device__ __forceinline__ void for_each_acc(const Core<MT, NT, WM, WN>& core, F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  using C = Core<MT, NT, WM, WN>;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        f((wm * C::FM + i) * 16 + 4 * (lane >> 4) + v, (wn * C::FN + j) * 16 + (lane & 15),
          core.acc[i][j][v]);
}

// ---------------------------------------------------------------------------
// Loaders
// ---------------------------------------------------------------------------

// bf16 rows contiguous along the reduction.  Two segments: steps [0, steps0)
// read p0 (leading dimension ld0, reduction extent k0), later steps read p1.
// Rows >= rows and reduction columns >= the segment's extent read as zero
// (extents are multiples of 8).
template <int R>
struct RowLoader {
  static constexpr int PER = R * 8 / 256;  // 16-byte chunks per thread
  const uint16_t *p0, *p1;
  int64_t ld0, ld1, k0, k1, rows;
  int steps0;
  u32x4_t v[PER];

  __device__ void load(int s) {
    const uint16_t* p = s < steps0 ? p0 : p1;
    const int64_t ld = s < steps0 ? ld0 : ld1;
    const int64_t kext = s < steps0 ? k0 : k1;
    const int64_t kb = (int64_t)(s < steps0 ? s : s - steps0) * KS;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int id = threadIdx.x + 256 * i;
      const int row = id >> 3, c = id & 7;
      const int64_t col = kb + 8 * c;
      if (row < rows && col < kext)
        v[i] = *reinterpret_cast<const u32x4_t*>(p + row * ld + col);
      else
        v[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* t) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int id = threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4_t*>(t + swz(id >> 3, id & 7)) = v[i];
    }
  }
};

// bf16 matrix L[m][p] (p contiguous, leading dimension ld) read with the
// reduction over m: tile rows are p (R of them, R = 64 or 128).  Each thread
// owns 8 consecutive m by R/32 consecutive p, transposed on the way into LDS.
// Rows m >= m_end and columns p >= P read as zero.
template <int R>
struct TransLoader {
  static constexpr int PPT = R / 32;  // p per thread
  static_assert(PPT == 2 || PPT == 4, "tile rows");
  const uint16_t* L;
  int64_t ld, P, p0, m_begin, m_end;
  uint32_t v[8][PPT / 2];

  __device__ void load(int step) {
    const int mg = threadIdx.x >> 5, pg = threadIdx.x & 31;
    const int64_t p = p0 + PPT * pg;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m_begin + (int64_t)step * KS + mg * 8 + i;
      const bool ok = m < m_end && p < P;
      if constexpr (PPT == 4) {
        u32x2_t t{0u, 0u};
        if (ok) t = *reinterpret_cast<const u32x2_t*>(L + m * ld + p);
        v[i][0] = t[0];
        v[i][1] = t[1];
      } else {
        v[i][0] = ok ? *reinterpret_cast<const uint32_t*>(L + m * ld + p) : 0u;
      }
    }
  }
  __device__ void store(char* t) const {
    const int mg = threadIdx.x >> 5, pg = threadIdx.x & 31;
#pragma unroll
    for (int kk = 0; kk < PPT; ++kk) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t wd = v[i][kk >> 1];
        h[i] = (kk & 1) ? (wd >> 16) : (wd & 0xffffu);
      }
      const u32x4_t o{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16)};
      *reinterpret_cast<u32x4_t*>(t + swz(PPT * pg + kk, mg)) = o;
    }
  }
};

// Like run_tiles, with a second tile of one operand (the low half of a bf16
// hi/lo pair): every step accumulates A·B and A2·B (SECOND_ON_A) or A·B and
// A·B2, i.e. the product with (hi + lo).
template <int MT, int NT, int WM, int WN, bool SECOND_ON_A, class LA, class LB, class L2>
__device__ __forceinline__ void run_tiles_pair(Core<MT, NT, WM, WN>& core, LA& la, LB& lb, L2& l2,
                                               int nsteps, char* smem) {
  constexpr int A_BYTES = MT * ROW_BYTES, B_BYTES = NT * ROW_BYTES;
  constexpr int X_BYTES = SECOND_ON_A ? A_BYTES : B_BYTES;
  constexpr int STAGE = A_BYTES + B_BYTES + X_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  core.zero();
  if (nsteps <= 0) return;
  auto sA = [&](int b) { return smem + b * STAGE; };
  auto sB = [&](int b) { return smem + b * STAGE + A_BYTES; };
  auto sX = [&](int b) { return smem + b * STAGE + A_BYTES + B_BYTES; };
  la.load(0);
  lb.load(0);
  l2.load(0);
  la.store(sA(0));
  lb.store(sB(0));
  l2.store(sX(0));
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      la.load(s + 1);
      lb.load(s + 1);
      l2.load(s + 1);
    }
    core.step(sA(cur), sB(cur), wm, wn, lane);
    if (SECOND_ON_A)
      core.step(sX(cur), sB(cur), wm, wn, lane);
    else
      core.step(sA(cur), sX(cur), wm, wn, lane);
    if (more) {
      la.store(sA(cur ^ 1));
      lb.store(sB(cur ^ 1));
      l2.store(sX(cur ^ 1));
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void split_hilo(float v, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = pack_bf16x2(v, 0.0f) & 0xffffu;
  const float rem = __fsub_rn(v, __uint_as_float(h << 16));
  hi = (uint16_t)h;
  lo = (uint16_t)(pack_bf16x2(rem, 0.0f) & 0xffffu);
}

__device__ __forceinline__ void load_codebook_lds(float* sq, const Codebook& cb) {
  if (threadIdx.x < 16) sq[threadIdx.x] = cb.q[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Partial low-rank products over one reduction slice z (grid.z):
//   kind 0:  P[z][m][j] = Σ_{k in slice} X[m][k] · A[j][k]       (T = X·Aᵀ)
//   kind 1:  P[z][m][j] = Σ_{n in slice} dY[m][n] · B2[n][j]      (U = dY·B)
// with j < Rp; B2 is the padded copy [N, 2Rp] of B.  Grid
// (ceil(M/128), ceil(Rp/64), slices); 128 x 64 tile, slices of `chunk`.
template <int KIND>
__global__ __launch_bounds__(256) void lora_partial_kernel(const uint16_t* __restrict__ L, int64_t M,
                                                           int64_t red, const uint16_t* __restrict__ R,
                                                           int r, int64_t Rp, int64_t chunk,
                                                           float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (128 + 64) * ROW_BYTES];
  const int64_t m0 = (int64_t)blockIdx.x * 128, j0 = (int64_t)blockIdx.y * 64;
  const int64_t c0 = (int64_t)blockIdx.z * chunk;
  int64_t cext = red - c0;
  if (cext > chunk) cext = chunk;
  RowLoader<128> la;
  la.p0 = la.p1 = L + m0 * red + c0;
  la.ld0 = la.ld1 = red;
  la.k0 = la.k1 = cext;
  la.rows = M - m0;
  la.steps0 = 1 << 30;
  Core<128, 64, 2, 2> core;
  const int nsteps = cext > 0 ? (int)((cext + KS - 1) / KS) : 0;
  if constexpr (KIND == 0) {
    RowLoader<64> lb;  // rows j of A [r, K]; rows >= r read as zero
    lb.p0 = lb.p1 = R + j0 * red + c0;
    lb.ld0 = lb.ld1 = red;
    lb.k0 = lb.k1 = cext;
    lb.rows = r - j0;
    lb.steps0 = 1 << 30;
    run_tiles(core, la, lb, nsteps, smem);
  } else {
    (void)r;
    TransLoader<64> lb;  // B2[n][j]: tile rows j, reduction n
    lb.L = R;
    lb.ld = 2 * Rp;
    lb.P = Rp;
    lb.p0 = j0;
    lb.m_begin = c0;
    lb.m_end = c0 + cext;
    run_tiles(core, la, lb, nsteps, smem);
  }
  float* o = P + blockIdx.z * M * Rp;
  for_each_acc(core, [&](int i, int jj, float v) {
    const int64_t m = m0 + i, j = j0 + jj;
    if (m < M && j < Rp) o[m * Rp + j] = v;
  });
}

// T[m][j] = Σ_z P[z][m][j] (fixed order); optional fp32 T [M, r]; and the
// hi/lo bf16 split of s·T into out [M, 2Rp] (zeros for j >= r).
__global__ void lora_reduce_kernel(const float* __restrict__ P, int S, int64_t M, int r, int64_t Rp,
                                   float scale, float* __restrict__ T, uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * Rp) return;
  const int64_t m = idx / Rp, j = idx % Rp;
  float acc = 0.0f;
  for (int z = 0; z < S; ++z) acc = __fadd_rn(acc, P[(int64_t)z * M * Rp + idx]);
  uint16_t hi = 0, lo = 0;
  if (j < r) {
    if (T) T[m * r + j] = acc;
    split_hilo(__fmul_rn(scale, acc), hi, lo);
  }
  out[m * 2 * Rp + j] = hi;
  out[m * 2 * Rp + Rp + j] = lo;
}

// sT from a saved fp32 T [M, r].
__global__ void split_saved_kernel(const float* __restrict__ T, int64_t M, int r, int64_t Rp,
                                   float scale, uint16_t* __restrict__ sT) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * Rp) return;
  const int64_t m = idx / Rp, j = idx % Rp;
  uint16_t hi = 0, lo = 0;
  if (j < r) split_hilo(__fmul_rn(scale, T[m * r + j]), hi, lo);
  sT[m * 2 * Rp + j] = hi;
  sT[m * 2 * Rp + Rp + j] = lo;
}

// dA partials:  P[z][j][k] = Σ_{m in slice} (sU_hi + sU_lo)[m][j] · X[m][k]
// Grid (ceil(K/128), ceil(Rp/64), slices); 64 x 128 tile.
__global__ __launch_bounds__(256) void da_partial_kernel(const uint16_t* __restrict__ sU, int64_t M,
                                                         int64_t Rp, const uint16_t* __restrict__ X,
                                                         int64_t K, int64_t chunk,
                                                         float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (64 + 128 + 64) * ROW_BYTES];
  const int64_t j0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 128;
  const int64_t mb = (int64_t)blockIdx.z * chunk;
  int64_t me = mb + chunk;
  if (me > M) me = M;
  TransLoader<64> la;   // hi half
  la.L = sU;
  la.ld = 2 * Rp;
  la.P = Rp;
  la.p0 = j0;
  la.m_begin = mb;
  la.m_end = me;
  TransLoader<64> la2 = la;  // lo half: columns Rp .. 2Rp
  la2.L = sU + Rp;
  TransLoader<128> lb;
  lb.L = X;
  lb.ld = K;
  lb.P = K;
  lb.p0 = k0;
  lb.m_begin = mb;
  lb.m_end = me;
  Core<64, 128, 2, 2> core;
  const int nsteps = me > mb ? (int)((me - mb + KS - 1) / KS) : 0;
  run_tiles_pair<64, 128, 2, 2, true>(core, la, lb, la2, nsteps, smem);
  float* o = P + blockIdx.z * Rp * K;
  for_each_acc(core, [&](int i, int jj, float v) {
    const int64_t j = j0 + i, k = k0 + jj;
    if (j < Rp && k < K) o[j * K + k] = v;
  });
}

// dB partials:  P[z][n][j] = Σ_{m in slice} dY[m][n] · (sT_hi + sT_lo)[m][j]
// Grid (ceil(Rp/64), ceil(N/128), slices); 128 x 64 tile.
__global__ __launch_bounds__(256) void db_partial_kernel(const uint16_t* __restrict__ dY, int64_t M,
                                                         int64_t N, const uint16_t* __restrict__ sT,
                                                         int64_t Rp, int64_t chunk,
                                                         float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (128 + 64 + 64) * ROW_BYTES];
  const int64_t n0 = (int64_t)blockIdx.y * 128, j0 = (int64_t)blockIdx.x * 64;
  const int64_t mb = (int64_t)blockIdx.z * chunk;
  int64_t me = mb + chunk;
  if (me > M) me = M;
  TransLoader<128> la;
  la.L = dY;
  la.ld = N;
  la.P = N;
  la.p0 = n0;
  la.m_begin = mb;
  la.m_end = me;
  TransLoader<64> lb;  // hi half
  lb.L = sT;
  lb.ld = 2 * Rp;
  lb.P = Rp;
  lb.p0 = j0;
  lb.m_begin = mb;
  lb.m_end = me;
  TransLoader<64> lb2 = lb;
  lb2.L = sT + Rp;
  Core<128, 64, 2, 2> core;
  const int nsteps = me > mb ? (int)((me - mb + KS - 1) / KS) : 0;
  run_tiles_pair<128, 64, 2, 2, false>(core, la, lb, lb2, nsteps, smem);
  float* o = P + blockIdx.z * N * Rp;
  for_each_acc(core, [&](int i, int jj, float v) {
    const int64_t n = n0 + i, j = j0 + jj;
    if (n < N && j < Rp) o[n * Rp + j] = v;
  });
}

// out[p][q] = Σ_z P[z·zs + p·Qp + q] for p < Pn, q < qv (fixed order z = 0..S-1);
// out is [Pn, qv].  With S == 0 it writes zeros.
__global__ void reduce_slices_kernel(const float* __restrict__ P, int S, int64_t zs, int64_t Pn,
                                     int64_t Qp, int64_t qv, float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Pn * qv) return;
  const int64_t p = idx / qv, q = idx % qv;
  float acc = 0.0f;
  for (int z = 0; z < S; ++z) acc = __fadd_rn(acc, P[(int64_t)z * zs + p * Qp + q]);
  out[idx] = acc;
}

unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// The forward GEMM lives in fwd.hip, the dX GEMM in dx.hip, the M <= 16
// forward path in gemv.hip.
hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* A, int32_t r, int64_t Rp, uint16_t* AT2, void* dX,
                          bool dx_bf16, hipStream_t st);
hipError_t launch_pad_lora_b(const uint16_t* B, int64_t N, int32_t r, int64_t Rp, uint16_t* B2,
                             hipStream_t st);
hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B, int32_t r, int64_t Rp, uint16_t* B2, void* Y,
                           bool y_bf16, hipStream_t st);
hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float scale, void* Y, bool y_bf16, float* T,
                       hipStream_t st);

// Slices of a long reduction so that a grid of `tiles` output tiles reaches
// about 512 workgroups; each slice is a multiple of 64 and at least 256 long.
static int64_t slice_len(int64_t red, int64_t tiles) {
  if (tiles < 1) tiles = 1;
  int64_t want = (512 + tiles - 1) / tiles;
  int64_t len = round_up((red + want - 1) / want, KS);
  if (len < 4 * KS) len = 4 * KS;
  return len;
}

FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  FwdLayout L{};
  const int64_t Rp = lora_rp(r);
  size_t off = 0;
  L.off_T = off;
  off += round_up(M * r * 4, 256);
  L.off_sT = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_B2 = off;
  off += M > 16 ? round_up(N * 2 * Rp * 2, 256) : 0;
  L.off_P = off;
  if (M > 16) {
    const int64_t tiles = cdiv(M, 128) * cdiv(Rp, 64);
    L.sliceT = slice_len(K, tiles);
    off += round_up(cdiv(K, L.sliceT) * M * Rp * 4, 256);
  }
  L.total = off;
  return L;
}

BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdLayout L{};
  const int64_t Rp = lora_rp(r);
  const int64_t mt = cdiv(M, 128) * cdiv(Rp, 64);
  L.sliceT = slice_len(K, mt);
  L.sliceU = slice_len(N, mt);
  L.sliceA = slice_len(M, cdiv(K, 128) * cdiv(Rp, 64));
  L.sliceB = slice_len(M, cdiv(N, 128) * cdiv(Rp, 64));
  size_t off = 0;
  L.off_sT = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_sU = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_B2 = off;
  off += round_up(N * 2 * Rp * 2, 256);
  L.off_AT2 = off;
  off += round_up(K * 2 * Rp * 2, 256);
  // one scratch area reused by the successive partial-sum kernels
  L.off_P = off;
  size_t p = 0;
  p = std::max<size_t>(p, round_up(cdiv(K, L.sliceT) * M * Rp * 4, 256));
  p = std::max<size_t>(p, round_up(cdiv(N, L.sliceU) * M * Rp * 4, 256));
  p = std::max<size_t>(p, round_up(cdiv(M, L.sliceA) * Rp * K * 4, 256));
  p = std::max<size_t>(p, round_up(cdiv(M, L.sliceB) * N * Rp * 4, 256));
  off += p;
  L.total = off;
  return L;
}

// T = X·Aᵀ (fp32 into T if non-null) and out = hi/lo(s·T).
static hipError_t lora_down(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int32_t r,
                            int64_t Rp, float scale, int64_t slice, float* P, float* T,
                            uint16_t* out, hipStream_t st) {
  const int64_t S = cdiv(K, slice);
  lora_partial_kernel<0><<<dim3(cdiv(M, 128), cdiv(Rp, 64), (unsigned)S), 256, 0, st>>>(
      X, M, K, A, r, Rp, slice, P);
  lora_reduce_kernel<<<cdiv(M * Rp, 256), 256, 0, st>>>(P, (int)S, M, r, Rp, scale, T, out);
  return hipGetLastError();
}

hipError_t launch_forward(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                          const uint16_t* B, int32_t r, float scale, void* Y, bool y_bf16,
                          float* T, char* ws, const FwdLayout& L, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (M <= 16) {
    float* Tw = T ? T : reinterpret_cast<float*>(ws + L.off_T);
    return launch_gemv(W, X, M, A, B, r, scale, Y, y_bf16, Tw, st);
  }
  const int64_t Rp = lora_rp(r);
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  hipError_t e = lora_down(X, M, W.K, A, r, Rp, scale, L.sliceT,
                           reinterpret_cast<float*>(ws + L.off_P), T, sT, st);
  if (e != hipSuccess) return e;
  uint16_t* B2 = reinterpret_cast<uint16_t*>(ws + L.off_B2);
  return launch_fwd_gemm(W, X, M, sT, B, r, Rp, B2, Y, y_bf16, st);
}

hipError_t launch_backward(const Nf4View& W, const uint16_t* X, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                           const float* T_saved, void* dX, bool dx_bf16, float* dA, float* dB,
                           char* ws, const BwdLayout& L, hipStream_t st) {
  const int64_t Rp = lora_rp(r);
  const int64_t N = W.N, K = W.K;
  float* P = reinterpret_cast<float*>(ws + L.off_P);
  if (M == 0) {
    reduce_slices_kernel<<<cdiv((int64_t)r * K, 256), 256, 0, st>>>(P, 0, 0, r, K, K, dA);
    reduce_slices_kernel<<<cdiv(N * r, 256), 256, 0, st>>>(P, 0, 0, N, Rp, r, dB);
    return hipGetLastError();
  }
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  uint16_t* sU = reinterpret_cast<uint16_t*>(ws + L.off_sU);
  uint16_t* B2 = reinterpret_cast<uint16_t*>(ws + L.off_B2);
  uint16_t* AT2 = reinterpret_cast<uint16_t*>(ws + L.off_AT2);
  hipError_t e;
  // s·T (hi/lo): from the saved T, or recomputed
  if (T_saved) {
    split_saved_kernel<<<cdiv(M * Rp, 256), 256, 0, st>>>(T_saved, M, r, Rp, scale, sT);
  } else {
    e = lora_down(X, M, K, A, r, Rp, scale, L.sliceT, P, nullptr, sT, st);
    if (e != hipSuccess) return e;
  }
  // s·U (hi/lo), U = dY·B
  e = launch_pad_lora_b(B, N, r, Rp, B2, st);
  if (e != hipSuccess) return e;
  {
    const int64_t S = cdiv(N, L.sliceU);
    lora_partial_kernel<1><<<dim3(cdiv(M, 128), cdiv(Rp, 64), (unsigned)S), 256, 0, st>>>(
        dY, M, N, B2, r, Rp, L.sliceU, P);
    lora_reduce_kernel<<<cdiv(M * Rp, 256), 256, 0, st>>>(P, (int)S, M, r, Rp, scale, nullptr, sU);
  }
  // dX = [dY | sU] · [Ŵ ; A ; A]
  e = launch_dx_gemm(W, dY, M, sU, A, r, Rp, AT2, dX, dx_bf16, st);
  if (e != hipSuccess) return e;
  // dA = Σ_m (sU_hi + sU_lo)ᵀ X  (s is already inside sU)
  {
    const int64_t S = cdiv(M, L.sliceA);
    da_partial_kernel<<<dim3(cdiv(K, 128), cdiv(Rp, 64), (unsigned)S), 256, 0, st>>>(
        sU, M, Rp, X, K, L.sliceA, P);
    reduce_slices_kernel<<<cdiv((int64_t)r * K, 256), 256, 0, st>>>(P, (int)S, Rp * K, r, K, K,
                                                                     dA);
  }
  // dB = Σ_m dYᵀ (sT_hi + sT_lo)
  {
    const int64_t S = cdiv(M, L.sliceB);
    db_partial_kernel<<<dim3(cdiv(Rp, 64), cdiv(N, 128), (unsigned)S), 256, 0, st>>>(
        dY, M, N, sT, Rp, L.sliceB, P);
    reduce_slices_kernel<<<cdiv(N * r, 256), 256, 0, st>>>(P, (int)S, N * Rp, N, Rp, r, dB);
  }
  return hipGetLastError();
}

}  // namespace qnf4
