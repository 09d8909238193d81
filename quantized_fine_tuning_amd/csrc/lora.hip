// Low-rank side products of the QLoRA linear layer, gfx950.
//
// P1 §七 (dataflow figure): the LoRA path runs beside the frozen 4-bit base,
// its output added to the base product.  P1 简化版 and P2 §4.4: the backward
// pass sends the gradient through the dequantized base into the adapters
// only.  With Y = X·Ŵᵀ + s·(X·Aᵀ)·Bᵀ and T = X·Aᵀ, U = dY·B:
//   forward:  T                      (reduction over the input features K)
//   backward: U                      (reduction over the output features N)
//             dA = s·Uᵀ·X  [r, K]    (reduction over the tokens M)
//             dB = s·dYᵀ·T [N, r]    (reduction over the tokens M)
// Each streams one large operand (X or dY) once against a small one, so
// the products are bound by HBM bandwidth and by how many bytes are in
// flight.  Two kernels cover them:
//   * rowred: P[z][m][j] = Σ_k L[m][k]·R[j][k] over slice z of k (T, U), both
//     operands contiguous along the reduction;
//   * colred: P[z][p][j] = Σ_m L[m][p]·S[j][m] over slice z of m (dA, dB),
//     with S = hi + lo rows of the transposed bf16 split of s·U or s·T.
// Both copy their operand tiles straight from global memory into a ring of
// four LDS stages (buffer loads with the LDS destination), three stages in
// flight per workgroup.  The stages are separate LDS arrays and the loop is
// unrolled over them, so that the compiler can tell the copy into one stage
// from the reads of another and needs no full wait before each read; each
// wave waits for its own copies of a stage before the barrier that opens it.
// Partial sums over the reduction slices are added in a fixed order by the
// reduction kernels below, which also produce the bf16 hi/lo splits.
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int ST = 64;     // reduction elements per stage
constexpr int NSTAGE = 4;  // ring depth

__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Barrier between stages: the waits that precede it are the caller's; the
// empty asm statements keep every LDS access on its side.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until the copies of the current stage are done: two more stages'
// copies (PER load instructions per stage and wave) may stay in flight.
template <int PER>
__device__ __forceinline__ void wait_stage() {
  wait_vmem_le<2 * PER>();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void split_hilo(float v, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = pack_bf16x2(v, 0.0f) & 0xffffu;
  const float rem = __fsub_rn(v, __uint_as_float(h << 16));
  hi = (uint16_t)h;
  lo = (uint16_t)(pack_bf16x2(rem, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// rowred: P[z][m][j0 + j] = Σ_{k in slice z} L[m][k] · R[j0 + j][k],  j < 64.
// L [M, Kred] (leading dimension ldl), R [rrows, Kred] (leading dimension
// ldr); rows past M or rrows read as zero, and so do reduction columns past
// Kred.  Workgroup: 64 rows of L by 64 rows of R, 4 waves of 32 x 32.
// Grid (ceil(M/64), ceil(Rp/64), slices of `chunk`).  Output [S, M, Rp].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rowred_kernel(const uint16_t* __restrict__ L, int64_t M,
                                                     int64_t Kred, int64_t ldl,
                                                     const uint16_t* __restrict__ R, int64_t rrows,
                                                     int64_t ldr, int64_t chunk, int64_t Rp,
                                                     float* __restrict__ P) {
  __shared__ __attribute__((aligned(1024))) char l0[64 * 128], l1[64 * 128], l2[64 * 128], l3[64 * 128];
  __shared__ __attribute__((aligned(1024))) char r0[64 * 128], r1[64 * 128], r2[64 * 128], r3[64 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 64;
  const int64_t kb = (int64_t)blockIdx.z * chunk;
  const int64_t kext = std::min(chunk, Kred - kb);
  const int nsteps = (int)((kext + ST - 1) / ST);

  // Resources start at (first row, kb); rows past the tensor are outside.
  const int64_t lbytes = ((M - m0) * ldl - kb) * 2, rbytes = ((rrows - j0) * ldr - kb) * 2;
  const rsrc_t rl = make_rsrc(L + m0 * ldl + kb, lbytes);
  const rsrc_t rr = make_rsrc(R + j0 * ldr + kb, rrows > j0 ? rbytes : 0);
  // Wave w copies rows 16w + 8c + (lane >> 3), c = 0, 1, of both tiles; lane
  // i fills physical chunk i & 7, i.e. logical chunk (i & 7) ^ (i >> 3).
  const int lch = (lane & 7) ^ (lane >> 3);
  const int crow = 16 * wave + (lane >> 3);
  const uint32_t vl = (uint32_t)((crow * ldl + 8 * lch) * 2), vr = (uint32_t)((crow * ldr + 8 * lch) * 2);
  const uint32_t l_oob = (uint32_t)std::min<int64_t>(std::max<int64_t>(lbytes, 0), 0x7fffffff);
  const uint32_t r_oob = (uint32_t)std::min<int64_t>(std::max<int64_t>(rbytes, 0), 0x7fffffff);

  // Steps past the slice are issued too, with every lane outside the
  // resource: they fill their stage with zeros, so that the pipeline has no
  // branches (a branch would make the compiler wait for all copies before
  // each LDS read) and the extra steps add nothing.
  auto issue = [&](char* lt, char* rt, int s) __attribute__((always_inline)) {
    const bool in = (int64_t)s * ST + 8 * lch < kext;  // also false past the slice
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t ol = in ? vl + (uint32_t)(c * 8 * ldl * 2) + (uint32_t)s * (ST * 2) : l_oob;
      const uint32_t orr = in ? vr + (uint32_t)(c * 8 * ldr * 2) + (uint32_t)s * (ST * 2) : r_oob;
      buf_load_lds16(rl, lt + (16 * wave + 8 * c) * 128, ol, 0u);
      buf_load_lds16(rr, rt + (16 * wave + 8 * c) * 128, orr, 0u);
    }
  };

  const int wm = wave >> 1, wj = wave & 1;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const char* lt, const char* rt) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(lt + xswz(32 * wm + 16 * i + lr, 2 * kq + ks));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(rt + xswz(32 * wj + 16 * j + lr, 2 * kq + ks));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
    }
  };
  // one step on the ring stage (lt, rt); the stage refilled after the
  // barrier is the one read in the previous step
  auto step = [&](int s, char* lt, char* rt, char* lnext, char* rnext) __attribute__((always_inline)) {
    wait_stage<4>();
    stage_barrier();
    issue(lnext, rnext, s + NSTAGE - 1);
    compute(lt, rt);
  };
  issue(l0, r0, 0);
  issue(l1, r1, 1);
  issue(l2, r2, 2);
  for (int s = 0; s < nsteps; s += NSTAGE) {
    step(s, l0, r0, l3, r3);
    step(s + 1, l1, r1, l0, r0);
    step(s + 2, l2, r2, l1, r1);
    step(s + 3, l3, r3, l2, r2);
  }
  wait_vmem();  // no copy may land in LDS after the workgroup ends

  float* o = P + (int64_t)blockIdx.z * M * Rp;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + 32 * wm + 16 * i + 4 * kq + v, jj = j0 + 32 * wj + 16 * j + lr;
        if (m < M && jj < Rp) o[m * Rp + jj] = acc[i][j][v];
      }
}

// ---------------------------------------------------------------------------
// colred: P[z][p0 + p][j0 + j] = Σ_{m in slice z} L[m][p] · (S[j][m] + S[Rp + j][m])
// for p < 128, j < 64.  L [Mred, Pn] (leading dimension ldl); S [2Rp, lds]
// (the transposed hi/lo split, columns m >= Mred zero).  Rows m past Mred
// read as zero.  Workgroup: 128 columns of L by 64 rows of S, 4 waves of
// 32 x 64.  Grid (ceil(Pn/128), ceil(Rp/64), slices).  Output [S, Pn, Rp].
//
// The L tile keeps the natural layout (rows m of 256 bytes, 16-byte chunk c
// of row m at physical chunk c ^ 2((m >> 3) & 7)); an MFMA operand needs 8
// consecutive m of one column, gathered with 8 two-byte reads.  The chunk
// XOR puts the 4 row groups of one read instruction on different banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lswz(int row, int chunk) {
  return row * 256 + ((chunk ^ (((row >> 3) & 7) << 1)) << 4);
}

__global__ __launch_bounds__(256) void colred_kernel(const uint16_t* __restrict__ L, int64_t Mred,
                                                     int64_t Pn, int64_t ldl,
                                                     const uint16_t* __restrict__ S, int64_t lds,
                                                     int64_t Rp, int64_t chunk, float* __restrict__ P) {
  __shared__ __attribute__((aligned(1024))) char l0[64 * 256], l1[64 * 256], l2[64 * 256], l3[64 * 256];
  __shared__ __attribute__((aligned(1024))) char s0[128 * 128], s1[128 * 128], s2[128 * 128], s3[128 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * 128, j0 = (int64_t)blockIdx.y * 64;
  const int64_t mb = (int64_t)blockIdx.z * chunk;
  const int64_t mext = std::min(chunk, Mred - mb);
  const int nsteps = (int)((mext + ST - 1) / ST);

  const rsrc_t rl = make_rsrc(L + mb * ldl + p0, ((Mred - mb) * ldl - p0) * 2);
  const rsrc_t rs = make_rsrc(S + mb, (2 * Rp * lds - mb) * 2);
  // L tile: wave w copies rows 16w + 4c + (lane >> 4), c = 0..3; lane i fills
  // physical chunk i & 15.  S tile: wave w copies rows 32w + 8c + (lane >> 3)
  // (tile rows 0..63: hi rows j0 + t, 64..127: lo rows Rp + j0 + t - 64).
  const int lpc = lane & 15;
  uint32_t vl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = 16 * wave + 4 * c + (lane >> 4);
    vl[c] = (uint32_t)((row * ldl + 8 * (lpc ^ (((row >> 3) & 7) << 1))) * 2);
  }
  uint32_t vs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = 32 * wave + 8 * c + (lane >> 3);
    const int64_t srow = t < 64 ? j0 + t : Rp + j0 + (t - 64);
    const int sch = (lane & 7) ^ (t & 7);
    vs[c] = (uint32_t)((srow * lds + 8 * sch) * 2);
  }
  // steps past the slice read zeros (all lanes outside the resources)
  // (the test is made on a vector register: a uniform one would become a
  // branch)
  auto issue = [&](char* lt, char* st, int s) __attribute__((always_inline)) {
    const bool in = opaque(s) < nsteps;
    const uint32_t sl = (uint32_t)((int64_t)s * ST * ldl * 2), ss = (uint32_t)s * (ST * 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      buf_load_lds16(rl, lt + (16 * wave + 4 * c) * 256, in ? vl[c] : 0x7fffffffu, sl);
      buf_load_lds16(rs, st + (32 * wave + 8 * c) * 128, in ? vs[c] : 0x7fffffffu, ss);
    }
  };

  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const char* lt, const char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      u32x4_t a[2];
#pragma unroll
      for (int pf = 0; pf < 2; ++pf) {
        const int p = 32 * wave + 16 * pf + lr;
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 32 * mh + 8 * kq + i;
          h[i] = *reinterpret_cast<const uint16_t*>(lt + lswz(row, p >> 3) + 2 * (p & 7));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) a[pf][t] = h[2 * t] | (h[2 * t + 1] << 16);
      }
#pragma unroll
      for (int jf = 0; jf < 4; ++jf) {
        const u32x4_t bh = *reinterpret_cast<const u32x4_t*>(st + xswz(16 * jf + lr, 4 * mh + kq));
        const u32x4_t bl = *reinterpret_cast<const u32x4_t*>(st + xswz(64 + 16 * jf + lr, 4 * mh + kq));
#pragma unroll
        for (int pf = 0; pf < 2; ++pf) {
          acc[pf][jf] = mfma_16x16x32(a[pf], bh, acc[pf][jf]);
          acc[pf][jf] = mfma_16x16x32(a[pf], bl, acc[pf][jf]);
        }
      }
    }
  };
  auto step = [&](int s, char* lt, char* st, char* lnext, char* snext) __attribute__((always_inline)) {
    wait_stage<8>();
    stage_barrier();
    issue(lnext, snext, s + NSTAGE - 1);
    compute(lt, st);
  };
  issue(l0, s0, 0);
  issue(l1, s1, 1);
  issue(l2, s2, 2);
  for (int s = 0; s < nsteps; s += NSTAGE) {
    step(s, l0, s0, l3, s3);
    step(s + 1, l1, s1, l0, s0);
    step(s + 2, l2, s2, l1, s1);
    step(s + 3, l3, s3, l2, s2);
  }
  wait_vmem();

  float* o = P + (int64_t)blockIdx.z * Pn * Rp;
#pragma unroll
  for (int pf = 0; pf < 2; ++pf)
#pragma unroll
    for (int jf = 0; jf < 4; ++jf)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t p = p0 + 32 * wave + 16 * pf + 4 * kq + v, j = j0 + 16 * jf + lr;
        if (p < Pn && j < Rp) o[p * Rp + j] = acc[pf][jf][v];
      }
}

// ---------------------------------------------------------------------------
// Reductions of the slices (fixed order z = 0..S-1) and operand preparation
// ---------------------------------------------------------------------------

// From P [S, M, Rp]: optional fp32 T [M, r]; hi/lo split of scale·T into
// out [M, 2Rp] (hi in columns < Rp, lo from Rp; zeros for j >= r) and, if
// outT is non-null, its transpose outT [2Rp, Mp] (zeros for m >= M).
// One thread per (m, j), m < Mp.
__global__ void lora_reduce_kernel(const float* __restrict__ P, int S, int64_t M, int64_t Mp, int r,
                                   int64_t Rp, float scale, float* __restrict__ T,
                                   uint16_t* __restrict__ out, uint16_t* __restrict__ outT) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Mp * Rp) return;
  // m runs fastest inside a block of 64 so that the transposed stores coalesce
  const int64_t mblk = idx / (64 * Rp), rem = idx % (64 * Rp);
  const int64_t j = rem / 64, m = mblk * 64 + rem % 64;
  uint16_t hi = 0, lo = 0;
  if (m < M) {
    float acc = 0.0f;
    for (int z = 0; z < S; ++z) acc = __fadd_rn(acc, P[((int64_t)z * M + m) * Rp + j]);
    if (j < r) {
      if (T) T[m * r + j] = acc;
      split_hilo(__fmul_rn(scale, acc), hi, lo);
    }
    out[m * 2 * Rp + j] = hi;
    out[m * 2 * Rp + Rp + j] = lo;
  }
  if (outT) {
    outT[j * Mp + m] = hi;
    outT[(Rp + j) * Mp + m] = lo;
  }
}

// sT and its transpose from a saved fp32 T [M, r].
__global__ void split_saved_kernel(const float* __restrict__ T, int64_t M, int64_t Mp, int r, int64_t Rp,
                                   float scale, uint16_t* __restrict__ sT, uint16_t* __restrict__ sTT) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Mp * Rp) return;
  const int64_t mblk = idx / (64 * Rp), rem = idx % (64 * Rp);
  const int64_t j = rem / 64, m = mblk * 64 + rem % 64;
  uint16_t hi = 0, lo = 0;
  if (m < M) {
    if (j < r) split_hilo(__fmul_rn(scale, T[m * r + j]), hi, lo);
    sT[m * 2 * Rp + j] = hi;
    sT[m * 2 * Rp + Rp + j] = lo;
  }
  sTT[j * Mp + m] = hi;
  sTT[(Rp + j) * Mp + m] = lo;
}

// out[a][b] = Σ_z P[z·zs + a·sa + b·sb] for a < An, b < Bn (fixed order);
// with S == 0, zeros.
__global__ void reduce_slices_kernel(const float* __restrict__ P, int S, int64_t zs, int64_t An,
                                     int64_t Bn, int64_t sa, int64_t sb, float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= An * Bn) return;
  const int64_t a = idx / Bn, b = idx % Bn;
  float acc = 0.0f;
  for (int z = 0; z < S; ++z) acc = __fadd_rn(acc, P[(int64_t)z * zs + a * sa + b * sb]);
  out[idx] = acc;
}

// BT [Rp, Np] = Bᵀ for j < r, n < N; zeros elsewhere.  B is [N, r].
__global__ void transpose_lora_b_kernel(const uint16_t* __restrict__ B, int64_t N, int64_t Np, int r,
                                        int64_t Rp, uint16_t* __restrict__ BT) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Rp * Np) return;
  const int64_t j = idx / Np, n = idx % Np;
  BT[idx] = (j < r && n < N) ? B[n * r + j] : (uint16_t)0;
}

unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// Reduction slices for `tiles` output tiles over `red` reduction elements:
// about 256 workgroups in all, but at least 8 stages per slice where the
// reduction allows it.
LoraSlices lora_slices(int64_t red, int64_t tiles) {
  const int64_t steps = std::max<int64_t>(1, (red + ST - 1) / ST);
  int64_t s = std::max<int64_t>(1, (256 + tiles - 1) / std::max<int64_t>(tiles, 1));
  s = std::min(s, std::max<int64_t>(1, steps / 8));
  const int64_t per = (steps + s - 1) / s;
  LoraSlices out;
  out.chunk = per * ST;
  out.count = (steps + per - 1) / per;
  return out;
}

int64_t lora_mp(int64_t M) { return round_up(std::max<int64_t>(M, 1), 64); }

hipError_t launch_rowred(const uint16_t* L, int64_t M, int64_t Kred, int64_t ldl, const uint16_t* R,
                         int64_t rrows, int64_t ldr, int64_t Rp, const LoraSlices& sl, float* P,
                         hipStream_t st) {
  rowred_kernel<<<dim3(cdiv(M, 64), cdiv(Rp, 64), (unsigned)sl.count), 256, 0, st>>>(
      L, M, Kred, ldl, R, rrows, ldr, sl.chunk, Rp, P);
  return hipGetLastError();
}

hipError_t launch_colred(const uint16_t* L, int64_t Mred, int64_t Pn, int64_t ldl, const uint16_t* S,
                         int64_t lds, int64_t Rp, const LoraSlices& sl, float* P, hipStream_t st) {
  colred_kernel<<<dim3(cdiv(Pn, 128), cdiv(Rp, 64), (unsigned)sl.count), 256, 0, st>>>(
      L, Mred, Pn, ldl, S, lds, Rp, sl.chunk, P);
  return hipGetLastError();
}

hipError_t launch_lora_reduce(const float* P, int S, int64_t M, int32_t r, int64_t Rp, float scale,
                              float* T, uint16_t* out, uint16_t* outT, hipStream_t st) {
  const int64_t Mp = lora_mp(M);
  lora_reduce_kernel<<<cdiv(Mp * Rp, 256), 256, 0, st>>>(P, S, M, Mp, r, Rp, scale, T, out, outT);
  return hipGetLastError();
}

hipError_t launch_split_saved(const float* T, int64_t M, int32_t r, int64_t Rp, float scale,
                              uint16_t* sT, uint16_t* sTT, hipStream_t st) {
  const int64_t Mp = lora_mp(M);
  split_saved_kernel<<<cdiv(Mp * Rp, 256), 256, 0, st>>>(T, M, Mp, r, Rp, scale, sT, sTT);
  return hipGetLastError();
}

hipError_t launch_reduce_slices(const float* P, int S, int64_t zs, int64_t An, int64_t Bn, int64_t sa,
                                int64_t sb, float* out, hipStream_t st) {
  if (An * Bn == 0) return hipSuccess;
  reduce_slices_kernel<<<cdiv(An * Bn, 256), 256, 0, st>>>(P, S, zs, An, Bn, sa, sb, out);
  return hipGetLastError();
}

hipError_t launch_transpose_lora_b(const uint16_t* B, int64_t N, int32_t r, int64_t Rp, uint16_t* BT,
                                   hipStream_t st) {
  const int64_t Np = round_up(N, 64);
  transpose_lora_b_kernel<<<cdiv(Rp * Np, 256), 256, 0, st>>>(B, N, Np, r, Rp, BT);
  return hipGetLastError();
}

}  // namespace qnf4
