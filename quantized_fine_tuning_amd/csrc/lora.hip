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
// LDS stages (buffer loads with the LDS destination; 8 stages of 16 KB for
// rowred, 5 of 32 KB for colred), all but one in flight per workgroup.  The stages are separate LDS arrays and the loop is
// unrolled over them, so that the compiler can tell the copy into one stage
// from the reads of another and needs no full wait before each read; each
// wave waits for its own copies of a stage before the barrier that opens it.
// The work is split evenly over the workgroups (stream-K, below); partial
// sums are added in a fixed order by the finishing kernels, which also
// produce the bf16 hi/lo splits.
#include <algorithm>

#include "host.h"

namespace qnf4 {
namespace {

constexpr int ST = 64;      // reduction elements per stage
constexpr int kRowRing = 8;  // rowred ring depth (8 x 16 KB)
constexpr int kColRing = 5;  // colred ring depth (5 x 32 KB)

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

// Waits until the copies of the current stage are done: the NS - 2 stages
// issued after it (PER load instructions per stage and wave) may stay in
// flight.
template <int NS, int PER>
__device__ __forceinline__ void wait_stage() {
  wait_vmem_le<(NS - 2) * PER>();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Work split (stream-K).  A product has `tiles` output tiles, each a
// reduction of ns stages, cut into units of NS stages, NS the depth of the
// copy ring (ut units per tile; the
// stages of a last, partial unit past ns read zeros).  Workgroup g of G
// takes units [gU/G, (g+1)U/G) of the U = tiles·ut units in tile order, so
// every workgroup has the same amount of work whatever the number of tiles;
// the copy ring runs on across tile boundaries.  At the end of each tile
// it holds, a workgroup writes its partial sum into slot g - first(t) of
// that tile; the reduction kernels add the slots of a tile in slot order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t sk_begin(uint32_t g, uint32_t U, uint32_t G) {
  return (uint32_t)(((uint64_t)g * U) / G);
}
// the workgroup whose range holds unit u
__device__ __host__ inline uint32_t sk_owner(uint32_t u, uint32_t U, uint32_t G) {
  uint32_t g = (uint32_t)(((uint64_t)u * G) / U);
  while (g + 1 < G && (uint32_t)(((uint64_t)(g + 1) * U) / G) <= u) ++g;
  while (g > 0 && (uint32_t)(((uint64_t)g * U) / G) > u) --g;
  return g;
}

// ---------------------------------------------------------------------------
// rowred: tile (mb, jb) = Σ_k L[64mb + i][k] · R[64jb + j][k], i, j < 64.
// L [M, Kred] (leading dimension ldl), R [rrows, Kred] (leading dimension
// ldr); rows past M or rrows and columns past Kred read as zero.  Tile t =
// mb·jt + jb; 4 waves of 32 x 32.  Partial tiles [tiles, cmax, 64, 64].
// ---------------------------------------------------------------------------
template <bool F16>
__global__ __launch_bounds__(256) void rowred_kernel(const uint16_t* __restrict__ L, int64_t M,
                                                     int64_t Kred, int64_t ldl,
                                                     const uint16_t* __restrict__ R, int64_t rrows,
                                                     int64_t ldr, int jt, uint32_t ut, uint32_t U,
                                                     int cmax, float* __restrict__ P) {
  constexpr int NS = kRowRing;
  // the ring: separate arrays per stage (see the file comment)
  __shared__ __attribute__((aligned(1024))) char l0[8192], l1[8192], l2[8192], l3[8192], l4[8192], l5[8192],
      l6[8192], l7[8192];
  __shared__ __attribute__((aligned(1024))) char r0[8192], r1[8192], r2[8192], r3[8192], r4[8192], r5[8192],
      r6[8192], r7[8192];
  char* const ls[NS] = {l0, l1, l2, l3, l4, l5, l6, l7};
  char* const rs[NS] = {r0, r1, r2, r3, r4, r5, r6, r7};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  const uint32_t u0 = sk_begin(g, U, G), u1 = sk_begin(g + 1, U, G);

  // Wave w copies rows 16w + 8c + (lane >> 3), c = 0, 1, of both tiles; lane
  // i fills physical chunk i & 7, i.e. logical chunk (i & 7) ^ (i >> 3).
  const int lch = (lane & 7) ^ (lane >> 3);
  const int crow = 16 * wave + (lane >> 3);
  const uint32_t vl = (uint32_t)((crow * ldl + 8 * lch) * 2), vr = (uint32_t)((crow * ldr + 8 * lch) * 2);
  // Source of a unit: the resources of its tile and its first stage (past
  // the workgroup's range: a stage beyond every tile, so all lanes read
  // zeros).
  struct Src {
    rsrc_t rl, rr;
    int k0;
  };
  auto src = [&](uint32_t u) __attribute__((always_inline)) {
    const uint32_t uu = u < u1 ? u : u1 - 1;
    const uint32_t t = uu / ut;
    const int64_t mb = t / jt, jb = t % jt;
    Src o;
    o.rl = make_rsrc(L + 64 * mb * ldl, (M - 64 * mb) * ldl * 2);
    o.rr = make_rsrc(R + 64 * jb * ldr, rrows > 64 * jb ? (rrows - 64 * jb) * ldr * 2 : 0);
    o.k0 = u < u1 ? (int)(uu - t * ut) * NS : (1 << 24);
    return o;
  };
  auto issue = [&](char* lt, char* rt, const Src& sr, int i) __attribute__((always_inline)) {
    const int kc = (sr.k0 + i) * ST;
    const bool in = (int64_t)kc + 8 * lch < Kred;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t ol = in ? vl + (uint32_t)(c * 8 * ldl * 2) + (uint32_t)kc * 2u : 0x7fffffffu;
      const uint32_t orr = in ? vr + (uint32_t)(c * 8 * ldr * 2) + (uint32_t)kc * 2u : 0x7fffffffu;
      buf_load_lds16(sr.rl, lt + (16 * wave + 8 * c) * 128, ol, 0u);
      buf_load_lds16(sr.rr, rt + (16 * wave + 8 * c) * 128, orr, 0u);
    }
  };

  const int wm = wave >> 1, wj = wave & 1;
  f32x4_t acc[2][2];
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
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16<F16>(a[i], b[j], acc[i][j]);
    }
  };
  // one stage: wait for it, open it, refill the stage read before it, multiply
  auto step = [&](const char* lt, const char* rt, char* ln, char* rn, const Src& sr, int i)
      __attribute__((always_inline)) {
    wait_stage<NS, 4>();
    stage_barrier();
    issue(ln, rn, sr, i);
    compute(lt, rt);
  };

  Src cur = src(u0);
#pragma unroll
  for (int i = 0; i + 1 < NS; ++i) issue(ls[i], rs[i], cur, i);
  uint32_t u = u0;
  while (u < u1) {
    const uint32_t t = u / ut, ue = std::min(u1, (t + 1) * ut);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (; u < ue; ++u) {
      // stage i holds stage i of unit u; the stage refilled at position i
      // takes stage NS - 1 of unit u (i = 0) or stage i - 1 of unit u + 1
      const Src nxt = src(u + 1);
      step(ls[0], rs[0], ls[NS - 1], rs[NS - 1], cur, NS - 1);
#pragma unroll
      for (int i = 1; i < NS; ++i) step(ls[i], rs[i], ls[i - 1], rs[i - 1], nxt, i - 1);
      cur = nxt;
    }
    float* o = P + ((int64_t)t * cmax + (g - sk_owner(t * ut, U, G))) * (64 * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          o[(32 * wm + 16 * i + 4 * kq + v) * 64 + 32 * wj + 16 * j + lr] = acc[i][j][v];
  }
  wait_vmem();  // no copy may land in LDS after the workgroup ends
}

// ---------------------------------------------------------------------------
// colred: tile (pb, jb) = Σ_m L[m][128pb + p] · (S[64jb + j][m] + S[Rp + 64jb + j][m])
// for p < 128, j < 64.  L [Mred, Pn] (leading dimension ldl); S [2Rp, lds]
// (the transposed hi/lo split, columns m >= Mred zero).  Rows m past Mred
// read as zero.  Tile t = pb·jt + jb; 4 waves of 32 x 64.  Partial tiles
// [tiles, cmax, 128, 64].
//
// The L tile keeps the natural layout (rows m of 256 bytes, 16-byte chunk c
// of row m at physical chunk c ^ 2((m >> 3) & 7)); an MFMA operand needs 8
// consecutive m of one column, gathered with 8 two-byte reads.  The chunk
// XOR puts the 4 row groups of one read instruction on different banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lswz(int row, int chunk) {
  return row * 256 + ((chunk ^ (((row >> 3) & 7) << 1)) << 4);
}

// Both adapter gradients run in one launch: workgroups [0, g1) take job j0
// (dA), the rest job j1 (dB), each job with its own stream-K plan over its
// own workgroups.
template <bool F16>
__global__ __launch_bounds__(256) void colred_kernel(ColredJob j0, ColredJob j1, uint32_t g1) {
  constexpr int NS = kColRing;
  const bool second = blockIdx.x >= g1;
  const ColredJob J = second ? j1 : j0;
  const uint16_t* __restrict__ L = J.L;
  const uint16_t* __restrict__ S = J.S;
  float* __restrict__ P = J.P;
  const int64_t Mred = J.Mred, ldl = J.ldl, lds = J.lds, Rp = J.Rp;
  const int jt = J.jt, cmax = J.cmax;
  const uint32_t ut = J.ut, U = J.U;
  __shared__ __attribute__((aligned(1024))) char l0[16384], l1[16384], l2[16384], l3[16384], l4[16384];
  __shared__ __attribute__((aligned(1024))) char s0[16384], s1[16384], s2[16384], s3[16384], s4[16384];
  char* const ls[NS] = {l0, l1, l2, l3, l4};
  char* const ss[NS] = {s0, s1, s2, s3, s4};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, kq = lane >> 4;
  const uint32_t G = J.G, g = second ? blockIdx.x - g1 : blockIdx.x;
  const uint32_t u0 = sk_begin(g, U, G), u1 = sk_begin(g + 1, U, G);

  // L tile: wave w copies rows 16w + 4c + (lane >> 4), c = 0..3; lane i fills
  // physical chunk i & 15.  S tile: wave w copies rows 32w + 8c + (lane >> 3)
  // (tile rows 0..63: hi rows 64jb + t, 64..127: lo rows Rp + 64jb + t - 64).
  const int lpc = lane & 15;
  uint32_t vl[4], vs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = 16 * wave + 4 * c + (lane >> 4);
    vl[c] = (uint32_t)((row * ldl + 8 * (lpc ^ (((row >> 3) & 7) << 1))) * 2);
    const int t = 32 * wave + 8 * c + (lane >> 3);
    const int64_t srow = t < 64 ? t : Rp + (t - 64);
    vs[c] = (uint32_t)((srow * lds + 8 * ((lane & 7) ^ (t & 7))) * 2);
  }
  const rsrc_t rs = make_rsrc(S, 2 * Rp * lds * 2);
  struct Src {
    rsrc_t rl;
    uint32_t sbase;  // byte offset of the tile's first S row
    int k0;
  };
  auto src = [&](uint32_t u) __attribute__((always_inline)) {
    const uint32_t uu = u < u1 ? u : u1 - 1;
    const uint32_t t = uu / ut;
    const int64_t pb = t / jt, jb = t % jt;
    Src o;
    o.rl = make_rsrc(L + 128 * pb, (Mred * ldl - 128 * pb) * 2);
    o.sbase = (uint32_t)(64 * jb * lds * 2);
    o.k0 = u < u1 ? (int)(uu - t * ut) * NS : (1 << 20);
    return o;
  };
  // (the row test is made on a vector register: on a scalar one it would
  // become a branch, and a branch makes the compiler wait for every copy)
  auto issue = [&](char* lt, char* st, const Src& sr, int i) __attribute__((always_inline)) {
    const int ks = sr.k0 + i;
    const bool in = (int64_t)opaque(ks) * ST < Mred;
    const uint32_t ol = (uint32_t)((int64_t)ks * ST * ldl * 2), os = sr.sbase + (uint32_t)ks * (ST * 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      buf_load_lds16(sr.rl, lt + (16 * wave + 4 * c) * 256, in ? vl[c] + ol : 0x7fffffffu, 0u);
      buf_load_lds16(rs, st + (32 * wave + 8 * c) * 128, in ? vs[c] + os : 0x7fffffffu, 0u);
    }
  };

  f32x4_t acc[2][4];
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
          acc[pf][jf] = mfma16<F16>(a[pf], bh, acc[pf][jf]);
          acc[pf][jf] = mfma16<F16>(a[pf], bl, acc[pf][jf]);
        }
      }
    }
  };
  auto step = [&](const char* lt, const char* st, char* ln, char* sn, const Src& sr, int i)
      __attribute__((always_inline)) {
    wait_stage<NS, 8>();
    stage_barrier();
    issue(ln, sn, sr, i);
    compute(lt, st);
  };

  Src cur = src(u0);
#pragma unroll
  for (int i = 0; i + 1 < NS; ++i) issue(ls[i], ss[i], cur, i);
  uint32_t u = u0;
  while (u < u1) {
    const uint32_t t = u / ut, ue = std::min(u1, (t + 1) * ut);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (; u < ue; ++u) {
      const Src nxt = src(u + 1);
      step(ls[0], ss[0], ls[NS - 1], ss[NS - 1], cur, NS - 1);
#pragma unroll
      for (int i = 1; i < NS; ++i) step(ls[i], ss[i], ls[i - 1], ss[i - 1], nxt, i - 1);
      cur = nxt;
    }
    float* o = P + ((int64_t)t * cmax + (g - sk_owner(t * ut, U, G))) * (128 * 64);
#pragma unroll
    for (int pf = 0; pf < 2; ++pf)
#pragma unroll
      for (int jf = 0; jf < 4; ++jf)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          o[(32 * wave + 16 * pf + 4 * kq + v) * 64 + 16 * jf + lr] = acc[pf][jf][v];
  }
  wait_vmem();
}

// ---------------------------------------------------------------------------
// Reductions of the partial tiles (slot order) and operand preparation
// ---------------------------------------------------------------------------

// Slot range of tile t: partial tiles P[t][0 .. count).
__device__ __forceinline__ int sk_count(uint32_t t, uint32_t ut, uint32_t U, uint32_t G) {
  return (int)(sk_owner((t + 1) * ut - 1, U, G) - sk_owner(t * ut, U, G)) + 1;
}

// acc[e] = slot 0 + slot 1 + ... + slot cnt-1 of element threadIdx.x + 256e
// (slots SLOT floats apart), added in slot order; the loads of four slots
// are issued before their adds.
template <int E, int SLOT>
__device__ __forceinline__ void sum_slots(const float* __restrict__ pt, int cnt, float* acc) {
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int c = 0; c < cnt; c += 4) {
    float v[4][E];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // an existing slot whatever i, so that the loads are unconditional
      const int ci = c + i < cnt ? c + i : cnt - 1;
#pragma unroll
      for (int e = 0; e < E; ++e) v[i][e] = pt[(int64_t)ci * SLOT + threadIdx.x + 256 * e];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (c + i < cnt) acc[e] = __fadd_rn(acc[e], v[i][e]);
  }
}

// rowred tiles (64 m x 64 j) → optional fp32 T [M, r]; hi/lo split of
// scale·T into out [M, 2Rp] (hi in columns < Rp, lo from Rp; zeros for
// j >= r) and, if outT is non-null, its transpose outT [2Rp, Mp] (zeros for
// m >= M).  One workgroup of 256 per 32 rows of a tile (8 values a thread,
// each slot's 8 loads issued together).
template <bool F16>
__global__ __launch_bounds__(256) void rowred_finish_kernel(const float* __restrict__ P, int jt, uint32_t ut,
                                                            uint32_t U, uint32_t G, int cmax, int64_t M,
                                                            int64_t Mp, int r, int64_t Rp, float scale,
                                                            float* __restrict__ T, uint16_t* __restrict__ out,
                                                            uint16_t* __restrict__ outT,
                                                            const uint16_t* __restrict__ B, int64_t N,
                                                            uint16_t* __restrict__ B2, uint32_t pad_b0) {
  __shared__ uint32_t sh[64][33];  // hi | lo << 16 of (j, m), padded
  if (blockIdx.x >= pad_b0) {
    // blocks past the tiles' (only when B2 is given): the forward GEMM's
    // LoRA operand, in the same launch: B2[n][j] = B[n][j mod Rp] for
    // (j mod Rp) < r, else 0 ([N, 2Rp]); 8 consecutive j of one row per
    // lane (2Rp is a multiple of 64), one 16-byte store
    const uint32_t cpr = (uint32_t)(2 * Rp / 8);  // chunks per row
    const uint32_t idx = (blockIdx.x - pad_b0) * 256u + threadIdx.x;
    if (idx >= (uint32_t)N * cpr) return;
    const uint32_t n = idx / cpr, jc = (idx - n * cpr) * 8u;
    const uint16_t* br = B + (int64_t)n * r;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t jj = jc + (uint32_t)e, j = jj >= (uint32_t)Rp ? jj - (uint32_t)Rp : jj;
      w[e] = br[j < (uint32_t)r ? j : 0u];  // unconditional: the 8 loads in flight together
      if (j >= (uint32_t)r) w[e] = 0u;
    }
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = w[2 * e] | (w[2 * e + 1] << 16);
    *reinterpret_cast<u32x4_t*>(B2 + (int64_t)idx * 8) = o;
    return;
  }
  const uint32_t t = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int64_t m0 = (int64_t)(t / jt) * 64 + 32 * half, j0 = (int64_t)(t % jt) * 64;
  const int cnt = sk_count(t, ut, U, G);
  const float* pt = P + (int64_t)t * cmax * 4096 + 32 * half * 64;
  float acc[8];
  sum_slots<8, 4096>(pt, cnt, acc);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = threadIdx.x + 256 * e, i = idx >> 6, jj = idx & 63;
    const int64_t m = m0 + i, j = j0 + jj;
    uint16_t hi = 0, lo = 0;
    if (m < M && j < r) {
      if (T) T[m * r + j] = acc[e];
      split_hilo16<F16>(__fmul_rn(scale, acc[e]), hi, lo);
    }
    if (m < M && j < Rp) {
      out[m * 2 * Rp + j] = hi;
      out[m * 2 * Rp + Rp + j] = lo;
    }
    sh[jj][i] = (uint32_t)hi | ((uint32_t)lo << 16);
  }
  if (!outT) return;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = threadIdx.x + 256 * e, jj = idx >> 5, i = idx & 31;
    const int64_t m = m0 + i, j = j0 + jj;
    if (j < Rp && m < Mp) {
      const uint32_t v = sh[jj][i];
      outT[j * Mp + m] = (uint16_t)(v & 0xffffu);
      outT[(Rp + j) * Mp + m] = (uint16_t)(v >> 16);
    }
  }
}

// colred tiles (128 p x 64 j) → out [Pn, r] (out[p][j], transpose == 0) or
// out [r, Pn] (out[j][p], transpose == 1).  One workgroup of 256 per 32
// rows p of a tile; workgroups [0, b1) finish job f0, the rest job f1.
__global__ __launch_bounds__(256) void colred_finish_kernel(ColredFinishJob f0, ColredFinishJob f1, uint32_t b1,
                                                            int r) {
  __shared__ float sh[64][33];
  const bool second = blockIdx.x >= b1;
  const ColredFinishJob F = second ? f1 : f0;
  const float* __restrict__ P = F.P;
  float* __restrict__ out = F.out;
  const int jt = F.jt, cmax = F.cmax, transpose = F.transpose;
  const uint32_t ut = F.ut, U = F.U, G = F.G;
  const int64_t Pn = F.Pn;
  const uint32_t bid = second ? blockIdx.x - b1 : blockIdx.x;
  const uint32_t t = bid >> 2, q = bid & 3;
  const int64_t p0 = (int64_t)(t / jt) * 128 + 32 * q, j0 = (int64_t)(t % jt) * 64;
  const int cnt = sk_count(t, ut, U, G);
  const float* pt = P + (int64_t)t * cmax * 8192 + 32 * q * 64;
  float acc[8];
  sum_slots<8, 8192>(pt, cnt, acc);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = threadIdx.x + 256 * e, i = idx >> 6, jj = idx & 63;
    const int64_t p = p0 + i, j = j0 + jj;
    if (!transpose) {
      if (p < Pn && j < r) out[p * r + j] = acc[e];
    } else {
      sh[jj][i] = acc[e];
    }
  }
  if (!transpose) return;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = threadIdx.x + 256 * e, jj = idx >> 5, i = idx & 31;
    const int64_t p = p0 + i, j = j0 + jj;
    if (p < Pn && j < r) out[j * Pn + p] = sh[jj][i];
  }
}

// The backward pass's operand copies in one launch, each through 64 x 64
// tiles transposed in LDS, so that every global load and store of a wave
// covers whole rows of 64 consecutive 16-bit (or fp32) values.  Tile column
// block jb0 of jb = ceil(Rp / 64) within each row block.  Blocks [0, b1):
// sT [M, 2Rp] and its transpose sTT [2Rp, Mp] from a saved fp32 T [M, r]
// (no blocks when T is null); [b1, b2): BT [Rp, Np] = Bᵀ zero-padded;
// [b2, ...): AT2 [K, 2Rp], AT2[k][j] = A[j mod Rp][k] for (j mod Rp) < r,
// else 0.  Lane l of the block handles column l & 63 of rows
// 4i + (l >> 6), i = 0..15, the loads of all 16 rows issued together.
template <bool F16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ T, int64_t M, int64_t Mp,
                                                       int r, int64_t Rp, float scale, uint16_t* __restrict__ sT,
                                                       uint16_t* __restrict__ sTT, const uint16_t* __restrict__ B,
                                                       int64_t N, int64_t Np, uint16_t* __restrict__ BT,
                                                       const uint16_t* __restrict__ A, int64_t K,
                                                       uint16_t* __restrict__ AT2, unsigned b1, unsigned b2,
                                                       unsigned jb) {
  __shared__ uint32_t sh[64][65];  // sh[col][row] of the tile read in
  const unsigned b = blockIdx.x;
  const int col = threadIdx.x & 63, row = threadIdx.x >> 6;
  if (b < b1) {
    // rows m, columns j of T
    const int64_t m0 = (int64_t)(b / jb) * 64, j = (int64_t)(b % jb) * 64 + col;
    float tv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = m0 + 4 * i + row;
      const bool ok = m < M && j < r;
      tv[i] = T[ok ? m * r + j : 0];  // unconditional: all 16 loads in flight
      if (!ok) tv[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = m0 + 4 * i + row;
      uint16_t hi = 0, lo = 0;
      if (m < M && j < r) split_hilo16<F16>(__fmul_rn(scale, tv[i]), hi, lo);
      if (m < M && j < Rp) {
        sT[m * 2 * Rp + j] = hi;
        sT[m * 2 * Rp + Rp + j] = lo;
      }
      sh[col][4 * i + row] = (uint32_t)hi | ((uint32_t)lo << 16);
    }
    __syncthreads();
    const int64_t j0 = (int64_t)(b % jb) * 64, m = m0 + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t jj = j0 + 4 * i + row;
      if (jj < Rp && m < Mp) {
        const uint32_t v = sh[4 * i + row][col];
        sTT[jj * Mp + m] = (uint16_t)(v & 0xffffu);
        sTT[(Rp + jj) * Mp + m] = (uint16_t)(v >> 16);
      }
    }
  } else if (b < b2) {
    // rows n, columns j of B
    const unsigned bb = b - b1;
    const int64_t n0 = (int64_t)(bb / jb) * 64, j0 = (int64_t)(bb % jb) * 64;
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t n = n0 + 4 * i + row, j = j0 + col;
      const bool ok = n < N && j < r;
      v[i] = B[ok ? n * r + j : 0];
      if (!ok) v[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sh[col][4 * i + row] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t j = j0 + 4 * i + row, n = n0 + col;
      if (j < Rp && n < Np) BT[j * Np + n] = (uint16_t)sh[4 * i + row][col];
    }
  } else {
    // rows j, columns k of A
    const unsigned bb = b - b2;
    const int64_t k0 = (int64_t)(bb / jb) * 64, j0 = (int64_t)(bb % jb) * 64;
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t j = j0 + 4 * i + row, k = k0 + col;
      const bool ok = j < r && k < K;
      v[i] = A[ok ? j * K + k : 0];
      if (!ok) v[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sh[col][4 * i + row] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t k = k0 + 4 * i + row, j = j0 + col;
      if (k < K && j < Rp) {
        const uint16_t v = (uint16_t)sh[4 * i + row][col];
        AT2[k * 2 * Rp + j] = v;
        AT2[k * 2 * Rp + Rp + j] = v;
      }
    }
  }
}

// Zeros of the adapter gradients when there are no tokens.
__global__ void zero_kernel(float* __restrict__ a, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) a[idx] = 0.0f;
}

unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// Stream-K plan of a product with `tiles` output tiles of `ns` stages each.
SkPlan sk_plan(int64_t tiles, int64_t ns, int jt, int ring, uint32_t gmax) {
  SkPlan p{};
  p.jt = jt;
  p.tiles = tiles;
  p.ut = (uint32_t)std::max<int64_t>(1, (ns + ring - 1) / ring);
  p.U = (uint32_t)(tiles * p.ut);
  p.G = std::min<uint32_t>(p.U, gmax);
  p.cmax = 1;
  for (int64_t t = 0; t < tiles; ++t) {
    const int c = (int)(sk_owner((uint32_t)((t + 1) * p.ut - 1), p.U, p.G) -
                        sk_owner((uint32_t)(t * p.ut), p.U, p.G)) + 1;
    p.cmax = std::max(p.cmax, c);
  }
  return p;
}

SkPlan rowred_plan(int64_t M, int64_t Kred, int64_t Rp) {
  const int jt = (int)cdiv(Rp, 64);
  return sk_plan((int64_t)cdiv(M, 64) * jt, cdiv(Kred, ST), jt, kRowRing, kSkWorkgroups);
}
int64_t colred_tiles(int64_t Pn, int64_t Rp) { return (int64_t)cdiv(Pn, 128) * cdiv(Rp, 64); }
SkPlan colred_plan(int64_t Mred, int64_t Pn, int64_t Rp, uint32_t gmax) {
  const int jt = (int)cdiv(Rp, 64);
  return sk_plan(colred_tiles(Pn, Rp), cdiv(Mred, ST), jt, kColRing, gmax);
}
uint32_t colred_split(int64_t K, int64_t N, int64_t Rp) {
  // both products reduce over the same tokens, so their units are in the
  // ratio of their tiles, whatever M
  const int64_t ta = colred_tiles(K, Rp), tb = colred_tiles(N, Rp);
  const int64_t ga = (2 * (int64_t)kSkWorkgroups * ta + (ta + tb)) / (2 * (ta + tb));
  return (uint32_t)std::min<int64_t>(kSkWorkgroups - 1, std::max<int64_t>(1, ga));
}
size_t rowred_partial_bytes(const SkPlan& p) { return (size_t)p.tiles * p.cmax * 64 * 64 * 4; }
size_t colred_partial_bytes(const SkPlan& p) { return (size_t)p.tiles * p.cmax * 128 * 64 * 4; }

int64_t lora_mp(int64_t M) { return round_up(std::max<int64_t>(M, 1), 64); }

hipError_t launch_rowred(const uint16_t* L, int64_t M, int64_t Kred, int64_t ldl, const uint16_t* R,
                         int64_t rrows, int64_t ldr, const SkPlan& p, float* P, bool f16, hipStream_t st) {
  if (f16)
    rowred_kernel<true><<<p.G, 256, 0, st>>>(L, M, Kred, ldl, R, rrows, ldr, p.jt, p.ut, p.U, p.cmax, P);
  else
    rowred_kernel<false><<<p.G, 256, 0, st>>>(L, M, Kred, ldl, R, rrows, ldr, p.jt, p.ut, p.U, p.cmax, P);
  return hipGetLastError();
}

hipError_t launch_rowred_finish(const float* P, const SkPlan& p, int64_t M, int32_t r, int64_t Rp,
                                float scale, float* T, uint16_t* out, uint16_t* outT, const uint16_t* B,
                                int64_t N, uint16_t* B2, bool f16, hipStream_t st) {
  const uint32_t b0 = (uint32_t)(2 * p.tiles);
  const unsigned grid = b0 + (B2 ? cdiv(N * 2 * Rp / 8, 256) : 0u);
  if (f16)
    rowred_finish_kernel<true><<<grid, 256, 0, st>>>(P, p.jt, p.ut, p.U, p.G, p.cmax, M, lora_mp(M), r, Rp, scale, T,
                                                     out, outT, B, N, B2, b0);
  else
    rowred_finish_kernel<false><<<grid, 256, 0, st>>>(P, p.jt, p.ut, p.U, p.G, p.cmax, M, lora_mp(M), r, Rp, scale, T,
                                                      out, outT, B, N, B2, b0);
  return hipGetLastError();
}

hipError_t launch_colred(const ColredJob& a, const ColredJob& b, bool f16, hipStream_t st) {
  const unsigned grid = a.G + b.G;
  if (f16)
    colred_kernel<true><<<grid, 256, 0, st>>>(a, b, a.G);
  else
    colred_kernel<false><<<grid, 256, 0, st>>>(a, b, a.G);
  return hipGetLastError();
}

hipError_t launch_colred_finish(const ColredFinishJob& a, const ColredFinishJob& b, int32_t r, hipStream_t st) {
  const unsigned b1 = (unsigned)(4 * a.tiles), grid = b1 + (unsigned)(4 * b.tiles);
  colred_finish_kernel<<<grid, 256, 0, st>>>(a, b, b1, r);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const float* T, int64_t M, int32_t r, int64_t Rp, float scale, uint16_t* sT,
                           uint16_t* sTT, const uint16_t* B, int64_t N, uint16_t* BT, const uint16_t* A,
                           int64_t K, uint16_t* AT2, bool f16, hipStream_t st) {
  const int64_t Mp = lora_mp(M), Np = round_up(N, 64);
  const unsigned jb = cdiv(Rp, 64);
  const unsigned b1 = T ? cdiv(Mp, 64) * jb : 0u;
  const unsigned b2 = b1 + cdiv(Np, 64) * jb;
  const unsigned b3 = b2 + cdiv(K, 64) * jb;
  if (f16)
    bwd_prep_kernel<true><<<b3, 256, 0, st>>>(T, M, Mp, r, Rp, scale, sT, sTT, B, N, Np, BT, A, K, AT2, b1, b2, jb);
  else
    bwd_prep_kernel<false><<<b3, 256, 0, st>>>(T, M, Mp, r, Rp, scale, sT, sTT, B, N, Np, BT, A, K, AT2, b1, b2, jb);
  return hipGetLastError();
}

hipError_t launch_zero(float* a, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  zero_kernel<<<cdiv(n, 256), 256, 0, st>>>(a, n);
  return hipGetLastError();
}

}  // namespace qnf4
