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
// reduction over m: tile rows are p (R of them), each thread owns 8
// consecutive m by 4 consecutive p, transposed on the way into LDS.  Rows
// m >= m_end and columns p >= P read as zero.
template <int R>
struct TransLoader {
  static_assert(R == 128, "tile rows");
  const uint16_t* L;
  int64_t ld, P, p0, m_begin, m_end;
  u32x2_t v[8];

  __device__ void load(int step) {
    const int mg = threadIdx.x >> 5, pg = threadIdx.x & 31;
    const int64_t p = p0 + 4 * pg;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m_begin + (int64_t)step * KS + mg * 8 + i;
      if (m < m_end && p < P)
        v[i] = *reinterpret_cast<const u32x2_t*>(L + m * ld + p);
      else
        v[i] = u32x2_t{0u, 0u};
    }
  }
  __device__ void store(char* t) const {
    const int mg = threadIdx.x >> 5, pg = threadIdx.x & 31;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t wd = v[i][kk >> 1];
        h[i] = (kk & 1) ? (wd >> 16) : (wd & 0xffffu);
      }
      const u32x4_t o{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16)};
      *reinterpret_cast<u32x4_t*>(t + swz(4 * pg + kk, mg)) = o;
    }
  }
};

// LoRA factor B[n][j] (row stride r) read with the reduction over n, for
// U = dY·B: tile rows are j (64 of them), 8 n by 2 j per thread.
struct LoraBTransLoader {
  const uint16_t* B;
  int64_t N;
  int r, j0;
  uint32_t v[2][8];

  __device__ void load(int step) {
    const int ng = threadIdx.x >> 5, jg = threadIdx.x & 31;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = j0 + 2 * jg + jj;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t n = (int64_t)step * KS + ng * 8 + i;
        v[jj][i] = (n < N && j < r) ? (uint32_t)B[n * r + j] : 0u;
      }
    }
  }
  __device__ void store(char* t) const {
    const int ng = threadIdx.x >> 5, jg = threadIdx.x & 31;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const u32x4_t o{v[jj][0] | (v[jj][1] << 16), v[jj][2] | (v[jj][3] << 16),
                      v[jj][4] | (v[jj][5] << 16), v[jj][6] | (v[jj][7] << 16)};
      *reinterpret_cast<u32x4_t*>(t + swz(2 * jg + jj, ng)) = o;
    }
  }
};

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

// T[M, r] = X · Aᵀ (fp32, optional) and sT = hi/lo(s·T) [M, 2Rp] bf16.
// Grid (ceil(Rp/64), ceil(M/64)).
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ X, int64_t M,
                                                        int64_t K, const uint16_t* __restrict__ A,
                                                        int r, int64_t Rp, float scale,
                                                        float* __restrict__ T,
                                                        uint16_t* __restrict__ sT) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (64 + 64) * ROW_BYTES];
  const int64_t m0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  RowLoader<64> la;
  la.p0 = la.p1 = X + m0 * K;
  la.ld0 = la.ld1 = K;
  la.k0 = la.k1 = K;
  la.rows = M - m0;
  la.steps0 = 1 << 30;
  RowLoader<64> lb;
  lb.p0 = lb.p1 = A + j0 * K;
  lb.ld0 = lb.ld1 = K;
  lb.k0 = lb.k1 = K;
  lb.rows = r - j0;
  lb.steps0 = 1 << 30;
  Core<64, 64, 2, 2> core;
  run_tiles(core, la, lb, (int)(K / KS), smem);
  for_each_acc(core, [&](int i, int jj, float v) {
    const int64_t m = m0 + i, j = j0 + jj;
    if (m < M && j < Rp) {
      uint16_t hi = 0, lo = 0;
      if (j < r) {
        if (T) T[m * r + j] = v;
        split_hilo(__fmul_rn(scale, v), hi, lo);
      }
      sT[m * 2 * Rp + j] = hi;
      sT[m * 2 * Rp + Rp + j] = lo;
    }
  });
}

// sU = hi/lo(s · dY·B) [M, 2Rp].  Grid (ceil(Rp/64), ceil(M/64)).
__global__ __launch_bounds__(256) void lora_up_kernel(const uint16_t* __restrict__ dY, int64_t M,
                                                      int64_t N, const uint16_t* __restrict__ B,
                                                      int r, int64_t Rp, float scale,
                                                      uint16_t* __restrict__ sU) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (64 + 64) * ROW_BYTES];
  const int64_t m0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  RowLoader<64> la;
  la.p0 = la.p1 = dY + m0 * N;
  la.ld0 = la.ld1 = N;
  la.k0 = la.k1 = N;
  la.rows = M - m0;
  la.steps0 = 1 << 30;
  LoraBTransLoader lb;
  lb.B = B;
  lb.N = N;
  lb.r = r;
  lb.j0 = (int)j0;
  Core<64, 64, 2, 2> core;
  run_tiles(core, la, lb, (int)((N + KS - 1) / KS), smem);
  for_each_acc(core, [&](int i, int jj, float v) {
    const int64_t m = m0 + i, j = j0 + jj;
    if (m < M && j < Rp) {
      uint16_t hi = 0, lo = 0;
      if (j < r) split_hilo(__fmul_rn(scale, v), hi, lo);
      sU[m * 2 * Rp + j] = hi;
      sU[m * 2 * Rp + Rp + j] = lo;
    }
  });
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

// C_z[P, Q] = Σ_{m in slice z} L[m][p] · Rm[m][q], fp32 partials.
// Grid (ceil(Q/128), ceil(P/128), slices).
__global__ __launch_bounds__(256) void tn_partial_kernel(const uint16_t* __restrict__ L, int64_t ldl,
                                                         int64_t P, const uint16_t* __restrict__ Rm,
                                                         int64_t ldr, int64_t Q, int64_t M,
                                                         int64_t m_per, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (128 + 128) * ROW_BYTES];
  const int64_t p0 = (int64_t)blockIdx.y * 128, q0 = (int64_t)blockIdx.x * 128;
  const int64_t mb = (int64_t)blockIdx.z * m_per;
  int64_t me = mb + m_per;
  if (me > M) me = M;
  TransLoader<128> la;
  la.L = L;
  la.ld = ldl;
  la.P = P;
  la.p0 = p0;
  la.m_begin = mb;
  la.m_end = me;
  TransLoader<128> lb;
  lb.L = Rm;
  lb.ld = ldr;
  lb.P = Q;
  lb.p0 = q0;
  lb.m_begin = mb;
  lb.m_end = me;
  Core<128, 128, 2, 2> core;
  const int nsteps = me > mb ? (int)((me - mb + KS - 1) / KS) : 0;
  run_tiles(core, la, lb, nsteps, smem);
  float* o = out + blockIdx.z * P * Q;
  for_each_acc(core, [&](int i, int j, float v) {
    const int64_t p = p0 + i, q = q0 + j;
    if (p < P && q < Q) o[p * Q + q] = v;
  });
}

// dA[j][k] = Σ_z (pA[z][j][k] + pA[z][Rp+j][k]);  pA is [S][2Rp][K].
__global__ void reduce_dA_kernel(const float* __restrict__ pA, int S, int64_t Rp, int r, int64_t K,
                                 float* __restrict__ dA) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)r * K) return;
  const int64_t j = idx / K, k = idx % K;
  float acc = 0.0f;
  for (int z = 0; z < S; ++z) {
    const float* p = pA + (int64_t)z * 2 * Rp * K;
    acc = __fadd_rn(acc, __fadd_rn(p[j * K + k], p[(Rp + j) * K + k]));
  }
  dA[idx] = acc;
}

// dB[n][j] = Σ_z (pB[z][n][j] + pB[z][n][Rp+j]);  pB is [S][N][2Rp].
__global__ void reduce_dB_kernel(const float* __restrict__ pB, int S, int64_t N, int64_t Rp, int r,
                                 float* __restrict__ dB) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * r) return;
  const int64_t n = idx / r, j = idx % r;
  float acc = 0.0f;
  for (int z = 0; z < S; ++z) {
    const float* p = pB + (int64_t)z * N * 2 * Rp;
    acc = __fadd_rn(acc, __fadd_rn(p[n * 2 * Rp + j], p[n * 2 * Rp + Rp + j]));
  }
  dB[idx] = acc;
}

unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// The forward GEMM lives in fwd.hip, the dX GEMM in dx.hip, the M <= 16
// forward path in gemv.hip.
hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* A, int32_t r, int64_t Rp, uint16_t* AT2, void* dX,
                          bool dx_bf16, hipStream_t st);
hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B, int32_t r, int64_t Rp, uint16_t* B2, void* Y,
                           bool y_bf16, hipStream_t st);
hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float scale, void* Y, bool y_bf16, float* T,
                       hipStream_t st);

FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  (void)K;
  FwdLayout L{};
  const int64_t Rp = lora_rp(r);
  size_t off = 0;
  L.off_T = off;
  off += round_up(M * r * 4, 256);
  L.off_sT = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_B2 = off;
  off += M > 16 ? round_up(N * 2 * Rp * 2, 256) : 0;
  L.total = off;
  return L;
}

static int64_t slices_for(int64_t M) {
  int64_t s = M / 512;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return s;
}

BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdLayout L{};
  const int64_t Rp = lora_rp(r);
  L.splitA = slices_for(M);
  L.splitB = slices_for(M);
  size_t off = 0;
  L.off_T = off;
  off += round_up(M * r * 4, 256);
  L.off_sT = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_sU = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_AT2 = off;
  off += round_up(K * 2 * Rp * 2, 256);
  L.off_pA = off;
  off += round_up(L.splitA * 2 * Rp * K * 4, 256);
  L.off_pB = off;
  off += round_up(L.splitB * N * 2 * Rp * 4, 256);
  L.total = off;
  return L;
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
  lora_down_kernel<<<dim3(cdiv(Rp, 64), cdiv(M, 64)), 256, 0, st>>>(X, M, W.K, A, r, Rp, scale, T,
                                                                   sT);
  uint16_t* B2 = reinterpret_cast<uint16_t*>(ws + L.off_B2);
  return launch_fwd_gemm(W, X, M, sT, B, r, Rp, B2, Y, y_bf16, st);
}

hipError_t launch_backward(const Nf4View& W, const uint16_t* X, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                           const float* T_saved, void* dX, bool dx_bf16, float* dA, float* dB,
                           char* ws, const BwdLayout& L, hipStream_t st) {
  const int64_t Rp = lora_rp(r);
  const int64_t N = W.N, K = W.K;
  float* pA = reinterpret_cast<float*>(ws + L.off_pA);
  float* pB = reinterpret_cast<float*>(ws + L.off_pB);
  if (M == 0) {
    reduce_dA_kernel<<<cdiv((int64_t)r * K, 256), 256, 0, st>>>(pA, 0, Rp, r, K, dA);
    reduce_dB_kernel<<<cdiv(N * r, 256), 256, 0, st>>>(pB, 0, N, Rp, r, dB);
    return hipGetLastError();
  }
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  uint16_t* sU = reinterpret_cast<uint16_t*>(ws + L.off_sU);
  if (T_saved) {
    split_saved_kernel<<<cdiv(M * Rp, 256), 256, 0, st>>>(T_saved, M, r, Rp, scale, sT);
  } else {
    lora_down_kernel<<<dim3(cdiv(Rp, 64), cdiv(M, 64)), 256, 0, st>>>(X, M, K, A, r, Rp, scale,
                                                                     nullptr, sT);
  }
  lora_up_kernel<<<dim3(cdiv(Rp, 64), cdiv(M, 64)), 256, 0, st>>>(dY, M, N, B, r, Rp, scale, sU);
  uint16_t* AT2 = reinterpret_cast<uint16_t*>(ws + L.off_AT2);
  hipError_t e = launch_dx_gemm(W, dY, M, sU, A, r, Rp, AT2, dX, dx_bf16, st);
  if (e != hipSuccess) return e;
  // dA' [2Rp, K] = sUᵀ · X ;  dB' [N, 2Rp] = dYᵀ · sT
  const int64_t mA = round_up((M + L.splitA - 1) / L.splitA, KS);
  tn_partial_kernel<<<dim3(cdiv(K, 128), cdiv(2 * Rp, 128), (unsigned)L.splitA), 256, 0, st>>>(
      sU, 2 * Rp, 2 * Rp, X, K, K, M, mA, pA);
  const int64_t mB = round_up((M + L.splitB - 1) / L.splitB, KS);
  tn_partial_kernel<<<dim3(cdiv(2 * Rp, 128), cdiv(N, 128), (unsigned)L.splitB), 256, 0, st>>>(
      dY, N, N, sT, 2 * Rp, 2 * Rp, M, mB, pB);
  reduce_dA_kernel<<<cdiv((int64_t)r * K, 256), 256, 0, st>>>(pA, (int)L.splitA, Rp, r, K, dA);
  reduce_dB_kernel<<<cdiv(N * r, 256), 256, 0, st>>>(pB, (int)L.splitB, N, Rp, r, dB);
  return hipGetLastError();
}

}  // namespace qnf4
