// Input gradient of the QLoRA linear layer, gfx950:
//   dX[M, K] = dY·Ŵ + s·U·A  =  [dY | sU_hi | sU_lo] · [Ŵ ; A ; A]
// (P1 简化版 and P2 §4.4: the gradient passes through the dequantized frozen
// weight; U = dY·B is the LoRA path's input gradient.)
//
// The reduction runs over the weight's rows n while the codes are contiguous
// along k, so the dequantized weight has to be transposed on its way to the
// MFMA B operand.  Design:
//   * 256x256 output tile per workgroup (token rows x input features) of 12
//     waves, three per SIMD, in two roles.  Waves 0..7 multiply: wave
//     (wm, wk) owns token rows [128wm, +128) and columns [64wk, +64), 64
//     v_mfma_f32_16x16x32_bf16 per 64-row reduction step, operands read from
//     LDS one MFMA group ahead.  Waves 8..11 (one per SIMD) produce: wave
//     8 + p copies a quarter of the next step's dY tile straight into LDS,
//     loads the codes of block column p (columns [64p, +64)) for the step
//     after and stores them transposed to LDS, and builds that block
//     column's 64 row tables a step ahead.
//   * The transposed bf16 tile Ŵᵀ[k][n] of a step is dequantized in 8 slices
//     of 32 columns: producer p takes slice 2p + 1, MFMA wave w < 4 takes
//     slice 2w after its MFMAs of the step before (waves 4..7, whose MFMAs
//     issue behind those of waves 0..3 on the same SIMDs, take none).
//   * Dequantization goes through a per-row table: for each weight row and
//     block one lane writes the 16 values RNE_bf16(fl32(q_j * c')) to LDS;
//     in a slice, lane (rg, cg) owns rows 8rg..8rg+7 by columns 4cg..4cg+3,
//     each code one 2-byte table read, and packs 8 consecutive rows of one
//     column into one 16-byte store: the values come out already
//     transposed.  Table slots, tile swizzles and lane maps are chosen so
//     that lookups, stores and fragment reads are free of LDS bank conflicts
//     (32 banks of 4 bytes; the measured conflict count is 32 cycles per
//     step, from 256 when 8 consecutive lanes stored to 4 chunk positions).
//     Rows past N get an all-zero table.
//   * The producers move the codes into LDS transposed as dwords: a lane
//     loads 16 bytes of each of two consecutive weight rows and stores, per
//     column group, both rows' 2 bytes with one byte permute (8 stores per
//     lane and step; 2-byte stores of one row at a time took 16 and cost
//     3-4% of the kernel).
//   * One barrier per step: after it the MFMA waves use dY(s) and Ŵᵀ(s)
//     while the other buffers fill with dY(s+1) and Ŵᵀ(s+1).
//   * The LoRA term is 2*Rp/64 extra steps with A = [sU_hi | sU_lo] and B from
//     AT2[k][j] = A[j mod Rp][k] (a transposed, padded copy of A), both
//     copied straight into LDS.
//   * With few tokens the tiles alone leave most compute units idle; then
//     the n steps are split over `splits` workgroups per tile (the last
//     split also takes the LoRA steps), each writing its fp32 partial tile
//     to P[split][M][K], summed in split order by splitk_reduce_kernel.
#include <type_traits>

#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TK = 256, NSTEP = 64;
constexpr int kMfmaWaves = 8, kProdWaves = 4, kWaves = kMfmaWaves + kProdWaves;
constexpr int kThreads = 64 * kWaves;

// Tiles are rows of 64 16-bit values (eight 16-byte chunks) whose chunks are
// XOR-permuted by bits of the row.  A fragment read gives the 64 lanes 16
// consecutive rows at 4 chunks; the permutations below let the gfx950 LDS
// serve it at its full 16-byte read rate (measured: 4 clocks per wave
// instruction, against 8 for c ^ (r & 7)).
// dY tile (token rows, 64 n each): chunk c of row r at physical
// c ^ sw(r & 7), sw swapping bits 0 and 1.
__device__ __forceinline__ int rsw(int row) { return ((row >> 1) & 1) | ((row & 1) << 1) | (row & 4); }
__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ rsw(row & 7)) << 4);
}
// Ŵᵀ tile (k rows, 64 n each): chunk c of row r at physical c ^ h(r) with
// h(r) = r3 | r1 << 1 | r2 << 2 (r_i = bit i of r).  Besides the fragment
// reads this also serves the dequantization stores (rows 4cg + c, cg =
// 0..7, at 8 chunks) at the LDS's write rate.
__device__ __forceinline__ int wsw(int row) { return ((row >> 3) & 1) | (row & 2) | (row & 4); }
__device__ __forceinline__ int wswz(int row, int chunk) {
  return row * 128 + ((chunk ^ wsw(row)) << 4);
}

// Lane of a dequantization slice -> (row group rg, column group cg):
// lane bits 0..5 are cg0, rg0, rg1, cg1, cg2, rg2.  Each half-wave then
// reads the tables of 4 row groups (32 banks once), and each 8 consecutive
// lanes store their 16-byte chunks to 8 distinct chunk positions.
__device__ __forceinline__ int dq_rg(int l) { return ((l >> 1) & 3) | ((l >> 3) & 4); }
__device__ __forceinline__ int dq_cg(int l) { return (l & 1) | ((l >> 2) & 6); }

template <int LSTEPS, bool F16>
__global__ __launch_bounds__(kThreads, 1) void dx_gemm_kernel(Nf4View W, const uint16_t* __restrict__ dY,
                                                              int64_t M, const uint16_t* __restrict__ sU,
                                                              const uint16_t* __restrict__ AT2,
                                                              int64_t Rp, void* __restrict__ dX,
                                                              int dx_bf16, int tiles_m, int tiles_k,
                                                              int splits, float* __restrict__ P,
                                                              Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sa0[TM * 128], sa1[TM * 128];  // A tiles: dY, then sU
  __shared__ __attribute__((aligned(16))) char sw[2][TK * 128];  // B tiles: Ŵᵀ, then AT2
  // per step slot: the row tables of each block column (row 8rg + i at
  // 256i + 32rg of its 2 KB), and the codes of each 32-column slice
  // transposed (the 2 bytes of columns 4cg..4cg+3 of row 8rg + i at byte 2i
  // of 16-byte slot 8rg + (cg ^ rg))
  __shared__ __attribute__((aligned(256))) char stab[2][4][64 * 32];
  __shared__ __attribute__((aligned(16))) char scode[2][8][64 * 16];
  int tmi, tki, sp;
  if (!tile_of(blockIdx.x, tiles_m, tiles_k, splits, tmi, tki, sp)) return;

  // (the wave index in a scalar register: the LDS addresses and offsets of
  // the copies derived from it are then formed by scalar instructions)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = dq_rg(lane), cg = dq_cg(lane);
  const int64_t K = W.K, N = W.N;
  const int64_t m0 = (int64_t)tmi * TM, k0 = (int64_t)tki * TK;
  // this workgroup's n steps [nfirst, nfirst + nsteps) (step indices below
  // are relative to nfirst) and its LoRA steps
  const int nall = (int)((N + NSTEP - 1) / NSTEP);
  const int nfirst = split_first(sp, splits, nall);
  const int nsteps = split_first(sp + 1, splits, nall) - nfirst;
  const int lsteps = sp == splits - 1 ? LSTEPS : 0;
  auto sab = [&](int i) { return i ? sa1 : sa0; };

  // Slice sigma (columns [32 sigma, +32)) of step t into Ŵᵀ(t): lane (rg, cg)
  // reads the codes of its rows and columns (row 2p in the low half of dword
  // p, row 2p + 1 in its high half), looks each up in its row's table and
  // stores column c of rows 8rg..8rg+7 at wswz(32 sigma + 4cg + c, rg) =
  // (st0 ^ 16(c & 2)) + 128c with st0 = wswz(32 sigma + 4cg, rg).  The
  // table of row 8rg + i sits at a 256-byte-aligned
  // base + 256i + 32rg, so a lookup address is base + 32rg with its low byte
  // replaced by 32rg | 2*code (one byte permute from codes pre-shifted four
  // at a time) plus the constant 256i.  Column pair cp2 = columns 2cp2,
  // 2cp2 + 1: with `overlap` (producers) the lookups of the second pair are
  // in flight while the first is packed and stored; the MFMA waves, short of
  // registers, keep one column's lookups in flight while the previous column
  // is packed and stored.
  const int code_rslot = 8 * rg + (cg ^ rg);
  const uint32_t rg32x4 = (uint32_t)rg * 0x20202020u;
  auto read_codes = [&](int t, int sigma) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4_t*>(scode[t & 1][sigma] + 16 * code_rslot);
  };
  auto lookup_cols = [&](uint32_t lb, const u32x4_t& we, const u32x4_t& wo, int cp2, uint32_t (*v)[8])
      __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t sel = 0x07060500u | (uint32_t)(2 * h + cp2);
        v[0][2 * p + h] = lds_read_u16(__builtin_amdgcn_perm(lb, we[p], sel) + 256u * (2 * p + h));
        v[1][2 * p + h] = lds_read_u16(__builtin_amdgcn_perm(lb, wo[p], sel) + 256u * (2 * p + h));
      }
  };
  // (the empty asm pins the wait for the lookups here: otherwise the values
  // are packed, and so waited for, right after the lookups are issued)
  auto store_cols = [&](char* dst, uint32_t st0, int cp2, uint32_t (*v)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      asm volatile("" : "+v"(v[cc][0]), "+v"(v[cc][1]), "+v"(v[cc][2]), "+v"(v[cc][3]), "+v"(v[cc][4]),
                   "+v"(v[cc][5]), "+v"(v[cc][6]), "+v"(v[cc][7]));
      const int c = 2 * cp2 + cc;
      u32x4_t o;
#pragma unroll
      for (int p = 0; p < 4; ++p) o[p] = v[cc][2 * p] | (v[cc][2 * p + 1] << 16);
      *reinterpret_cast<u32x4_t*>(dst + ((st0 ^ (uint32_t)(16 * (c & 2))) + 128u * c)) = o;
    }
  };
  auto dequant_slice = [&](auto overlap, int t, int sigma, const u32x4_t& cw, auto&& issue)
      __attribute__((always_inline)) {
    if constexpr (decltype(overlap)::value) {
      const uint32_t lb = lds_offset(stab[t & 1][sigma >> 1]) + 32u * (uint32_t)rg;
      const uint32_t st0 =
          (uint32_t)((32 * sigma + 4 * cg) * 128 + ((rg ^ ((cg >> 1) & 1) ^ (4 * (cg & 1))) << 4));
      u32x4_t we, wo;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        we[p] = ((cw[p] << 1) & 0x1E1E1E1Eu) | rg32x4;  // byte j: 2 * code 2j
        wo[p] = ((cw[p] >> 3) & 0x1E1E1E1Eu) | rg32x4;  // byte j: 2 * code 2j+1
      }
      uint32_t v0[2][8], v1[2][8];
      lookup_cols(lb, we, wo, 0, v0);
      issue(0);
      __builtin_amdgcn_sched_barrier(0x8 | 0x4 | 0x10);
      lookup_cols(lb, we, wo, 1, v1);
      issue(1);
      __builtin_amdgcn_sched_barrier(0x8 | 0x4 | 0x10);
      store_cols(sw[t & 1], st0, 0, v0);
      store_cols(sw[t & 1], st0, 1, v1);
    } else {
      // addresses straight from the code dwords and lane offsets recomputed
      // here from an opaque copy of the lane index (kept from being hoisted
      // out of the MFMA waves' loop, where they would hold registers through
      // the MFMAs)
      const int ln = opaque(lane), lrg = dq_rg(ln), lcg = dq_cg(ln);
      const uint32_t lb = lds_offset(stab[t & 1][sigma >> 1]) + 32u * (uint32_t)lrg;
      const uint32_t st0 =
          (uint32_t)((32 * sigma + 4 * lcg) * 128 + ((lrg ^ ((lcg >> 1) & 1) ^ (4 * (lcg & 1))) << 4));
      // column c + 1's lookups are issued before column c is packed and
      // stored; each lookup address leaves its row offset 256i to the
      // instruction's offset field (the opaque copy keeps the compiler from
      // folding it into eight per-row base registers, which the second
      // column's values need; ≈0.7 % on the kernel)
      auto look_col = [&](int c, uint32_t* v) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            v[2 * p + h] = lds_read_u16(opaque(lb | code_x2(cw[p], 16 * h + 4 * c)) + 256u * (2 * p + h));
      };
      uint32_t va[8], vb[8];
      look_col(0, va);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t* const v = (c & 1) ? vb : va;
        if (c < 3) look_col(c + 1, (c & 1) ? va : vb);
        issue(c);
        __builtin_amdgcn_sched_barrier(0x8 | 0x4 | 0x10);
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                     "+v"(v[7]));
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = v[2 * p] | (v[2 * p + 1] << 16);
        *reinterpret_cast<u32x4_t*>(sw[t & 1] + ((st0 ^ (uint32_t)(16 * (c & 2))) + 128u * c)) = o;
      }
    }
  };
  auto no_issue = [](int) {};

  if (wave < kMfmaWaves) {
    // ---------------------------------------------------------------- MFMA
    const int lr = lane & 15, kq = lane >> 4;
    const int wm = wave >> 2, wk = wave & 3;
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // MFMA group g (0..15) of a step: n-half ks = g / 8, token block i = g % 8.
    // A fragments are read one group ahead: group g first reads the A
    // fragment of group g + 1, so the read's latency overlaps this group's
    // MFMAs.  At a step's start the A fragment of group 0 is requested before
    // the four B fragments, so that its first MFMA waits for two reads, not
    // five (LDS reads return in order; about 1% on the step).  The B
    // fragments of the second n-half are read right after the MFMAs of
    // group 7.
    const int arow = 128 * wm + lr, brow = 64 * wk + lr;
    u32x4_t bfr[4], anext;
    auto read_b = [&](const char* wb, int ks, u32x4_t* b) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(wb + wswz(brow + 16 * j, 2 * kq + ks));
    };
    auto read_a = [&](const char* ya, int g) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4_t*>(ya + xswz(arow + 16 * (g & 7), 2 * kq + (g >> 3)));
    };
    auto mfma_step = [&](const char* ya, const char* wb) __attribute__((always_inline)) {
      anext = read_a(ya, 0);
      read_b(wb, 0, bfr);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int i = g & 7;
        const u32x4_t a = anext;
        if (g < 15) anext = read_a(ya, g + 1);
        // keep the reads ahead of the MFMAs (the scheduler would sink them
        // below to reuse the fragment's registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<F16>(a, bfr[j], acc[i][j]);
        if (g == 7) read_b(wb, 1, bfr);
      }
    };

    const bool dq = wave < 4;  // dequantizes slice 2w of every step
    __syncthreads();  // codes and tables of steps 0 and 1 in place
    auto read_codes_mfma = [&](int t) __attribute__((always_inline)) {
      const int ln = opaque(lane);
      return *reinterpret_cast<const u32x4_t*>(scode[t & 1][2 * wave] + 16 * (8 * dq_rg(ln) + (dq_cg(ln) ^ dq_rg(ln))));
    };
    if (dq) dequant_slice(std::false_type(), 0, 2 * wave, read_codes_mfma(0), no_issue);
    __syncthreads();  // step 0 in place
#pragma unroll 1
    for (int s = 0; s + 1 < nsteps; ++s) {
      mfma_step(sab(s & 1), sw[s & 1]);
      if (dq) dequant_slice(std::false_type(), s + 1, 2 * wave, read_codes_mfma(s + 1), no_issue);
      __syncthreads();
    }
#pragma unroll 1
    for (int s = nsteps - 1; s < nsteps + lsteps; ++s) {
      mfma_step(sab(s & 1), sw[s & 1]);
      __syncthreads();
    }

    // epilogue: lane holds rows 128wm + 16i + 4kq + v of column k0 + 64wk + 16j + lr
    int row0 = 128 * wm + 4 * kq, col0 = 64 * wk + lr;
    asm volatile("" : "+v"(row0), "+v"(col0));
    const bool full = (m0 + TM <= M) && (k0 + TK <= K);
    if (splits > 1) {
      float* Pp = P + ((int64_t)sp * M + m0 + row0) * K + k0 + col0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + row0 + 16 * i + v, k = k0 + col0 + 16 * j;
            if (full || (m < M && k < K)) Pp[(16 * i + v) * K + 16 * j] = acc[i][j][v];
          }
    } else if (dx_bf16) {
      uint16_t* D = static_cast<uint16_t*>(dX) + (m0 + row0) * K + k0 + col0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + row0 + 16 * i + v, k = k0 + col0 + 16 * j;
            if (full || (m < M && k < K))
              D[(16 * i + v) * K + 16 * j] = (uint16_t)(pack16<F16>(acc[i][j][v], 0.0f) & 0xffffu);
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
    return;
  }

  // ------------------------------------------------------------ producers
  const int p = wave - kMfmaWaves;
  const uint32_t kpr = (uint32_t)(K / kBlock);
  const uint32_t kb = (uint32_t)(k0 / kBlock) + (uint32_t)p;  // this producer's block column
  const bool cols_ok = k0 + 64 * p < K;
  const float mu = *W.mu;
  const rsrc_t rsu = make_rsrc(sU + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t rc = make_rsrc(W.codes, N * (K / 2));
  const rsrc_t re = make_rsrc(W.e, N * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rat = make_rsrc(AT2 + k0 * 2 * Rp, (K - k0) * 2 * Rp * 2);

  // dY rows [64p, +64) of a step, copied straight into LDS: part c moves rows
  // 64p + 8c + (l >> 3), lane l into physical chunk l & 7, so it fetches
  // logical chunk (l & 7) ^ sw(l >> 3) (row & 7 = l >> 3).  Each instruction
  // fills 1 KB of LDS contiguously.  (Written as assembly: the compiler then
  // inserts no wait for these copies in front of the producer's own LDS
  // reads; the wait before the step's closing barrier is explicit.)
  const int ylch = (lane & 7) ^ rsw(lane >> 3);
  const uint32_t vy = (uint32_t)(((64 * p + (lane >> 3)) * N + 8 * ylch) * 2);
  const uint32_t y_gstride = (uint32_t)(8 * N * 2);
  const i32x4_t ryw = rsrc_words(dY + m0 * N, (M - m0) * N * 2);
  auto copy_y_part = [&](char* t, int s, int c) __attribute__((always_inline)) {
    dma_lds16(ryw, t + (64 * p + 8 * c) * 128, vy + c * y_gstride, (uint32_t)(nfirst + s) * 128u);
  };
  auto copy_y = [&](char* t, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) copy_y_part(t, s, c);
  };
  // LoRA tiles, the same rows: sU rows in the xswz layout, AT2 rows in wswz.
  const uint32_t vsu = (uint32_t)(((64 * p + (lane >> 3)) * 2 * Rp + 8 * ylch) * 2);
  auto copy_su = [&](char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(rsu, t + (64 * p + 8 * c) * 128, vsu, c * (uint32_t)(8 * 2 * Rp * 2) + (uint32_t)l * 128u);
  };
  auto copy_at = [&](char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int row = 64 * p + 8 * c + (lane >> 3);
      const int lch = (lane & 7) ^ wsw(row);
      buf_load_lds16(rat, t + (64 * p + 8 * c) * 128, (uint32_t)((row * 2 * Rp + 8 * lch) * 2),
                     (uint32_t)l * 128u);
    }
  };

  // Codes of weight rows t*64 + 2m and 2m + 1 (m = lane & 31), columns
  // [64p + 32h, +32) of the tile (h = lane >> 5, slice 2p + h): 16 bytes of
  // each row.  A column group (4 columns, 2 bytes) of both rows is one
  // dword, stored at byte 4(m & 3) of slot 8rg + (cg ^ rg), rg = m >> 2: the
  // 32 lanes of each half-wave cover the 32 banks once.
  const int cm = lane & 31, ch = lane >> 5;
  const uint32_t vcode =
      (uint32_t)(2 * cm) * (uint32_t)(K / 2) + (uint32_t)(k0 / 2) + 32u * (uint32_t)p + 16u * (uint32_t)ch;
  const uint32_t code_sstride = (uint32_t)(NSTEP * (K / 2));
  struct Codes {
    u32x4_t c0, c1;
  };
  auto load_codes = [&](Codes& r, int t) __attribute__((always_inline)) {
    r.c0 = buf_load16(rc, vcode, (uint32_t)(nfirst + t) * code_sstride);
    r.c1 = buf_load16(rc, vcode + (uint32_t)(K / 2), (uint32_t)(nfirst + t) * code_sstride);
  };
  const int crg = cm >> 2;
  const uint32_t code_wbase = (uint32_t)(crg * 128 + 4 * (cm & 3));
  auto store_codes = [&](int t, const Codes& r) __attribute__((always_inline)) {
    char* const base = scode[t & 1][2 * p + ch];
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) {
      const uint32_t off = code_wbase + (uint32_t)(((pc ^ crg) & 7) << 4);
      *reinterpret_cast<uint32_t*>(base + off) =
          __builtin_amdgcn_perm(r.c1[pc >> 1], r.c0[pc >> 1], (pc & 1) ? 0x07060302u : 0x05040100u);
    }
  };

  // Table of row 8 tb_rg + tb_i of block column p with tb_rg = t0 + 2t1 + 4t3
  // and tb_i = t4 + 2t5 + 4t2 for lane t (t_b = bit b of t); the lane writes
  // half t2 of it first, so the 8 lanes of each 16-byte write cover a
  // 128-byte line.  Its e4m3 byte and group scale are loaded a step ahead.
  const int tb_rg = (lane & 3) | ((lane >> 1) & 4), tb_i = ((lane >> 4) & 3) | (lane & 4);
  const int tb_row = 8 * tb_rg + tb_i;
  const int tb_first = (lane >> 2) & 1;
  const int tb_off = 256 * tb_i + 32 * tb_rg + 16 * tb_first;
  struct Consts {
    uint32_t e, s;
  };
  auto load_consts = [&](Consts& r, int t) __attribute__((always_inline)) {
    const uint32_t blk = ((uint32_t)(nfirst + t) * NSTEP + (uint32_t)tb_row) * kpr + kb;
    r.e = buf_load1(re, blk, 0u);
    r.s = buf_load4(rs, (blk / kDqBlock) * 4u, 0u);
  };
  auto build_table = [&](int t, const Consts& r) __attribute__((always_inline)) {
    const bool row_ok = cols_ok && ((int64_t)(nfirst + t) * NSTEP + tb_row < N);
    const float cp = decode_constant(r.e, __uint_as_float(r.s), mu);
    u32x4_t t0, t1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t0[j] = row_ok ? pack16<F16>(__fmul_rn(cb.q[2 * j], cp), __fmul_rn(cb.q[2 * j + 1], cp)) : 0u;
      t1[j] = row_ok ? pack16<F16>(__fmul_rn(cb.q[8 + 2 * j], cp), __fmul_rn(cb.q[9 + 2 * j], cp)) : 0u;
    }
    char* const d = stab[t & 1][p] + tb_off;
    *reinterpret_cast<u32x4_t*>(d) = tb_first ? t1 : t0;
    *reinterpret_cast<u32x4_t*>((char*)((uintptr_t)d ^ 16u)) = tb_first ? t0 : t1;
  };

  Codes cn;
  Consts cc, cnx;
  // prologue: dY of step 0, codes and tables of steps 0 and 1, slice of step 0
  {
    Codes c0;
    Consts k0c;
    copy_y(sa0, 0);
    load_codes(c0, 0);
    load_codes(cn, 1);
    load_consts(k0c, 0);
    load_consts(cnx, 1);
    load_consts(cc, 2);
    store_codes(0, c0);
    store_codes(1, cn);
    build_table(0, k0c);
    build_table(1, cnx);
  }
  __syncthreads();  // codes and tables of steps 0 and 1 in place
  dequant_slice(std::true_type(), 0, 2 * p + 1, read_codes(0, 2 * p + 1), no_issue);
  wait_vmem();
  __syncthreads();  // step 0 in place

  // Reduction steps 0 .. nsteps-2: build the tables of step s+2 (that
  // buffer was last read in the previous iteration; the constants were
  // loaded then), then issue the copy of dY of step s+1 (first, so that it
  // has the whole step to land) and the loads of the codes of step s+2 and
  // the constants of step s+3, dequantize slice 2p + 1 of step s+1, then
  // store the codes of step s+2.  (The empty asm keeps the table's
  // arithmetic, and the compiler's wait for its constants, ahead of the
  // copies: the compiler does not track those, and a wait it places after
  // them would also wait for them.)
  // Weight data past the last step may be loaded: its reads stay inside the
  // buffers or return zeros, and it is not used.
#pragma unroll 1
  for (int s = 0; s + 1 < nsteps; ++s) {
    char* const yn = sab((s + 1) & 1);
    build_table(s + 2, cc);
    asm volatile("" ::: "memory");
    copy_y(yn, s + 1);
    load_codes(cn, s + 2);
    load_consts(cnx, s + 3);
    dequant_slice(std::true_type(), s + 1, 2 * p + 1, read_codes(s + 1, 2 * p + 1), no_issue);
    store_codes(s + 2, cn);
    cc = cnx;
    wait_vmem();
    __syncthreads();
  }
  // last reduction step: copy LoRA step 0 (sU and AT2 tiles) into the other
  // buffers; then the LoRA steps
  if (lsteps > 0) {
    copy_su(sab(nsteps & 1), 0);
    copy_at(sw[nsteps & 1], 0);
  }
  wait_vmem();
  __syncthreads();
#pragma unroll 1
  for (int l = 0; l < lsteps; ++l) {
    const int s = nsteps + l;
    if (l + 1 < lsteps) {
      copy_su(sab((s + 1) & 1), l + 1);
      copy_at(sw[(s + 1) & 1], l + 1);
    }
    wait_vmem();
    __syncthreads();
  }
}

}  // namespace

int dx_gemm_splits(int64_t M, int64_t N, int64_t K, size_t cap) {
  const int64_t tiles = ((M + TM - 1) / TM) * ((K + TK - 1) / TK);
  return gemm_splits(tiles, (N + NSTEP - 1) / NSTEP, M, K, cap);
}

hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* AT2, int64_t Rp, void* dX, bool dx16, int splits, float* P, bool f16,
                          hipStream_t st) {
  const int tm = (int)((M + TM - 1) / TM), tk = (int)((W.K + TK - 1) / TK);
  const unsigned grid = tile_grid(tm, tk, splits);
  const int db = dx16 ? 1 : 0;
  switch (2 * Rp / NSTEP) {
#define QNF4_DX_CASE(LS)                                                                      \
  case LS:                                                                                    \
    return f16 ? timed_launch(kKernDxGemm, dx_gemm_kernel<LS, true>, dim3(grid), dim3(kThreads), st, W, dY, M, \
                              (const uint16_t*)sU, (const uint16_t*)AT2, Rp, dX, db, tm, tk, splits, P, codebook()) \
               : timed_launch(kKernDxGemm, dx_gemm_kernel<LS, false>, dim3(grid), dim3(kThreads), st, W, dY, M, \
                              (const uint16_t*)sU, (const uint16_t*)AT2, Rp, dX, db, tm, tk, splits, P, codebook());
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
