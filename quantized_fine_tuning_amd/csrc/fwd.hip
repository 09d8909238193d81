// Forward product of the QLoRA linear layer for M > 16 tokens, gfx950:
//   Y[M, N] = X·Ŵᵀ + s·T·Bᵀ  =  [X | sT_hi | sT_lo] · [Ŵ | B | B]ᵀ
// (P1 §七 dataflow figure: the 4-bit base is dequantized to BF16 for the
// matmul and the LoRA path is added to the output.)
//
// Design
//   * 256x256 output tile per workgroup of 12 waves, three per SIMD, in two
//     roles.  Waves 0..7 only multiply: wave (wm, wn) owns token rows
//     [128wm, +128) and weight rows [64wn, +64) of the tile, 64
//     v_mfma_f32_16x16x32_bf16 per 64-wide reduction step, operands read
//     from LDS one MFMA group ahead.  Waves 8..11 (one per SIMD) produce the
//     operands: each copies a quarter of the next step's X tile straight
//     into LDS and dequantizes 64 of the tile's 256 weight rows of the next
//     step into the shared bf16 tile Ŵ[n][k].  The producers' table
//     arithmetic, lookups and copies overlap the MFMAs of the other two
//     waves of their SIMD instead of interrupting a wave's own MFMA stream.
//   * Dequantization goes through a per-row table: lane t writes the 16
//     values RNE_bf16(fl32(q_j * c')) of its row t to LDS, and every code is
//     one 2-byte table read (bit-identical to multiplying per element, since
//     the value depends only on code and row).  For row group q lane l reads
//     rows 8q + (l >> 3), k = 8(l & 7) + 0..7: the 8 lanes of one row hit its
//     table, and the 4 rows of each half-wave (served in one LDS cycle) hit 4
//     different groups of 8 of the 32 banks.  The lookups of one row group
//     are in flight while the previous group's values are packed and stored.
//   * Tiles are stored with 16-byte chunks XOR-swizzled by row (xswz) so that
//     MFMA operand reads of 8 rows cover the 32 LDS banks once.
//   * The packed codes, e4m3 bytes and group scales of step s+2 are loaded
//     while step s+1 is dequantized; codes go through LDS (each producer
//     reads back only its own rows), constants stay in registers.
//   * One barrier per step: after it the MFMA waves use X(s) and Ŵ(s) while
//     the producers fill the other buffers with X(s+1) and Ŵ(s+1).
//   * All operand reads are buffer loads whose resources end at the tensor's
//     last row, so ragged tiles read zeros without per-lane branches.
//   * The LoRA up-projection is 2*Rp/64 extra reduction steps whose A operand
//     is the bf16 hi/lo split of s·T and whose B operand is the padded copy
//     B2 = [B | 0 | B | 0] ([N, 2Rp] bf16), both copied straight into LDS.
//   * Workgroups are mapped to tiles so that each XCD (workgroup id mod 8)
//     walks a contiguous run of a grouped tile order (4 M-tiles per group):
//     the ~32 workgroups resident on one XCD share X and code rows in its L2.
//   * With few tokens the tiles alone leave most compute units idle; then
//     the K steps are split over `splits` workgroups per tile (the last
//     split also takes the LoRA steps), each writing its fp32 partial tile
//     to P[split][M][N], summed in split order by splitk_reduce_kernel.
#include <type_traits>

#include "host.h"
#include "tiling.h"

namespace qnf4 {
namespace {

constexpr int TM = 256, TN = 256, KSTEP = 64;
constexpr int kMfmaWaves = 8, kProdWaves = 4, kWaves = kMfmaWaves + kProdWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kProdRows = TN / kProdWaves;  // weight rows per producer wave

// A tile row = 64 bf16 = eight 16-byte chunks; chunk c of row r is stored at
// physical chunk c ^ sw(r & 7), where sw swaps bits 0 and 1 of its argument.
// An MFMA operand read gives the 64 lanes 16 consecutive rows at 4 chunks;
// with this permutation the gfx950 LDS serves it at its full 16-byte read
// rate (measured: 4 clocks per wave instruction), where the plain c ^ (r & 7)
// takes twice as long.  The write paths are indifferent to the choice.
__device__ __forceinline__ int rsw(int row) { return ((row >> 1) & 1) | ((row & 1) << 1) | (row & 4); }
__device__ __forceinline__ int xswz(int row, int chunk) {
  return row * 128 + ((chunk ^ rsw(row & 7)) << 4);
}

template <int LSTEPS, bool F16>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                               int64_t M, const uint16_t* __restrict__ sT,
                                                               const uint16_t* __restrict__ B2,
                                                               int64_t Rp, void* __restrict__ Y,
                                                               int y_bf16, int tiles_m, int tiles_n,
                                                               int splits, float* __restrict__ P,
                                                               Codebook cb) {
  __shared__ __attribute__((aligned(16))) char sx0[TM * 128], sx1[TM * 128];  // A tiles: X, then sT
  __shared__ __attribute__((aligned(16))) char sw[2][TN * 128];  // B tiles: Ŵ, then B2
  // tables of the tile's weight rows (row r at 32(r % 8) + 256(r / 8)),
  // double-buffered by step
  __shared__ __attribute__((aligned(256))) char stab[2][TN * 32];
  int tmi, tni, sp;
  if (!tile_of(blockIdx.x, tiles_m, tiles_n, splits, tmi, tni, sp)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t K = W.K, N = W.N;
  const int64_t m0 = (int64_t)tmi * TM, n0 = (int64_t)tni * TN;
  // this workgroup's K steps [kfirst, kfirst + ksteps) (step indices below
  // are relative to kfirst) and its LoRA steps
  const int kall = (int)(K / KSTEP);
  const int kfirst = split_first(sp, splits, kall);
  const int ksteps = split_first(sp + 1, splits, kall) - kfirst;
  const int lsteps = sp == splits - 1 ? LSTEPS : 0;
  auto sxb = [&](int i) { return i ? sx1 : sx0; };

  // Resources start at this tile's first row and end at the tensor's last
  // row: rows past M or N read as zero.  (Rows past M only feed output rows
  // past M, rows past N only output columns past N; neither is stored.)
  // Reads of weight data one or two steps past the last step stay inside
  // these buffers or return zeros; their results are never used.
  const rsrc_t rc = make_rsrc(W.codes + n0 * (K / 2), (N - n0) * (K / 2));

  // Lookups of a row group (8 weight rows from tile row R, a multiple of 8):
  // lane l = (dr, dc) = (l >> 3, l & 7) takes code dword dc of row R + dr
  // (k = 8dc .. 8dc + 7 of the step) and looks each code up in its row's
  // table, then stores the 8 bf16 as one 16-byte chunk.  The 8 lanes of a
  // row hit its table, and the 4 rows of each half-wave (served in one LDS
  // cycle) hit 4 different groups of 8 of the 32 banks.  The table of row
  // R + dr starts at a 256-byte-aligned base + 256(R / 8) + 32dr, so a
  // lookup address is that address with its low byte replaced by
  // 32dr | 2*code; the low bytes of the 4 even (odd) codes of a dword are
  // formed together, then each address is one byte permute.
  const int dr = lane >> 3, dc = lane & 7;
  const uint32_t dr32x4 = (uint32_t)dr * 0x20202020u;
  auto load_code = [&](int R, int t) __attribute__((always_inline)) {
    return buf_load4(rc, (uint32_t)(R + dr) * (uint32_t)(K / 2) + 4u * (uint32_t)dc, (uint32_t)(kfirst + t) * 32u);
  };
  auto lookup_group = [&](uint32_t w, const char* tabs, int R, uint32_t* v) __attribute__((always_inline)) {
    const uint32_t tab = lds_offset(tabs) + 256u * (uint32_t)(R >> 3) + 32u * (uint32_t)dr;
    const uint32_t we = ((w << 1) & 0x1E1E1E1Eu) | dr32x4;  // byte j: 2 * code 2j
    const uint32_t wo = ((w >> 3) & 0x1E1E1E1Eu) | dr32x4;  // byte j: 2 * code 2j+1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = lds_read_u16(__builtin_amdgcn_perm(tab, we, 0x07060500u | (uint32_t)j));
      v[2 * j + 1] = lds_read_u16(__builtin_amdgcn_perm(tab, wo, 0x07060500u | (uint32_t)j));
    }
  };
  // (the empty asm pins the wait for the lookups here: otherwise the values
  // are packed, and so waited for, right after the lookups are issued)
  auto store_group = [&](uint32_t* v, char* dst, int R) __attribute__((always_inline)) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                 "+v"(v[7]));
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = v[2 * j] | (v[2 * j + 1] << 16);
    *reinterpret_cast<u32x4_t*>(dst + xswz(R + dr, dc)) = o;
  };
  // NG row groups from R0 (8 rows apart), lookups of group q in flight while
  // group q - 1 is packed and stored; issue(q) runs after group q's lookups.
  auto dequant_rows = [&](auto NGc, int R0, const uint32_t* cw, int t, auto&& issue)
      __attribute__((always_inline)) {
    constexpr int NG = decltype(NGc)::value;
    uint32_t lv[2][8];
#pragma unroll
    for (int q = 0; q <= NG; ++q) {
      if (q < NG) {
        lookup_group(cw[q], stab[t & 1], R0 + 8 * q, lv[q & 1]);
        issue(q);
        __builtin_amdgcn_sched_barrier(0x8 | 0x4 | 0x10);
      }
      if (q > 0) store_group(lv[(q - 1) & 1], sw[t & 1], R0 + 8 * (q - 1));
    }
  };
  auto no_issue = [](int) {};

  if (wave < kMfmaWaves) {
    // ---------------------------------------------------------------- MFMA
    const int lr = lane & 15, kq = lane >> 4;
    const int wm = wave >> 2, wn = wave & 3;
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // MFMA group g (0..15) of a step: k-half ks = g / 8, token block i = g % 8.
    // A fragments are read one group ahead: group g first reads the A
    // fragment of group g + 1, so the read's latency overlaps this group's
    // MFMAs.  The B fragments of the second k-half are read right after the
    // MFMAs of group 7.
    const int arow = 128 * wm + lr, brow = 64 * wn + lr;
    u32x4_t bfr[4], anext;
    auto read_b = [&](const char* wb, int ks, u32x4_t* b) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(wb + xswz(brow + 16 * j, 2 * kq + ks));
    };
    auto read_a = [&](const char* xa, int g) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4_t*>(xa + xswz(arow + 16 * (g & 7), 2 * kq + (g >> 3)));
    };
    auto mfma_step = [&](const char* xa, const char* wb) __attribute__((always_inline)) {
      read_b(wb, 0, bfr);
      anext = read_a(xa, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int i = g & 7;
        const u32x4_t a = anext;
        if (g < 15) anext = read_a(xa, g + 1);
        // keep the reads ahead of the MFMAs (the scheduler would sink them
        // below to reuse the fragment's registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<F16>(a, bfr[j], acc[i][j]);
        if (g == 7) read_b(wb, 1, bfr);
      }
    };

    // This wave also dequantizes weight rows [16w, 16w + 16) of every step,
    // after its MFMAs of the step before.
    const int R0 = 16 * wave;
    uint32_t cw[2];
    cw[0] = load_code(R0, 0);
    cw[1] = load_code(R0 + 8, 0);
    __syncthreads();  // tables of steps 0 and 1 in place
    dequant_rows(std::integral_constant<int, 2>(), R0, cw, 0, no_issue);
    __syncthreads();  // step 0 in place
#pragma unroll 1
    for (int s = 0; s + 1 < ksteps; ++s) {
      cw[0] = load_code(R0, s + 1);
      cw[1] = load_code(R0 + 8, s + 1);
      mfma_step(sxb(s & 1), sw[s & 1]);
      dequant_rows(std::integral_constant<int, 2>(), R0, cw, s + 1, no_issue);
      __syncthreads();
    }
#pragma unroll 1
    for (int s = ksteps - 1; s < ksteps + lsteps; ++s) {
      mfma_step(sxb(s & 1), sw[s & 1]);
      __syncthreads();
    }

    // epilogue: lane holds rows 128wm + 16i + 4kq + v of column 64wn + 16j + lr.
    // The row/column bases go through an empty asm so that their address
    // arithmetic is not hoisted above the main loop (it would stay live there).
    int row0 = 128 * wm + 4 * kq, col0 = 64 * wn + lr;
    asm volatile("" : "+v"(row0), "+v"(col0));
    const bool full = (m0 + TM <= M) && (n0 + TN <= N);
    if (splits > 1) {
      float* Pp = P + ((int64_t)sp * M + m0 + row0) * N + n0 + col0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + row0 + 16 * i + v, n = n0 + col0 + 16 * j;
            if (full || (m < M && n < N)) Pp[(16 * i + v) * N + 16 * j] = acc[i][j][v];
          }
    } else if (y_bf16) {
      uint16_t* Yb = static_cast<uint16_t*>(Y) + (m0 + row0) * N + n0 + col0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + row0 + 16 * i + v, n = n0 + col0 + 16 * j;
            if (full || (m < M && n < N))
              Yb[(16 * i + v) * N + 16 * j] = (uint16_t)(pack16<F16>(acc[i][j][v], 0.0f) & 0xffffu);
          }
    } else {
      float* Yf = static_cast<float*>(Y) + (m0 + row0) * N + n0 + col0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + row0 + 16 * i + v, n = n0 + col0 + 16 * j;
            if (full || (m < M && n < N)) Yf[(16 * i + v) * N + 16 * j] = acc[i][j][v];
          }
    }
    return;
  }

  // ------------------------------------------------------------ producers
  // Producer p builds the tables of weight rows [64p, 64p + 64), dequantizes
  // rows [128 + 32p, +32) and copies X rows [64p, +64) of every step.
  const int p = wave - kMfmaWaves;
  const uint32_t kpr = (uint32_t)(K / kBlock);  // blocks per weight row
  const float mu = *W.mu;
  const rsrc_t rt = make_rsrc(sT + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t re = make_rsrc(W.e + n0 * kpr, (N - n0) * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rb = make_rsrc(B2 + n0 * 2 * Rp, (N - n0) * 2 * Rp * 2);

  // X rows [64p, +64) of a step, copied straight into LDS: part c
  // moves rows 64p + 8c + (l >> 3), lane l into physical chunk l & 7, so it
  // fetches logical chunk (l & 7) ^ sw(l >> 3) (row & 7 = l >> 3).  Each
  // instruction fills 1 KB of LDS contiguously.  (Written as assembly: the
  // compiler then inserts no wait for these copies in front of the
  // producer's own LDS reads; the wait before the step's closing barrier is
  // explicit.)
  const int xlch = (lane & 7) ^ rsw(lane >> 3);
  const uint32_t vx = (uint32_t)(((64 * p + (lane >> 3)) * K + 8 * xlch) * 2);
  const uint32_t x_gstride = (uint32_t)(8 * K * 2);
  const i32x4_t rxw = rsrc_words(X + m0 * K, (M - m0) * K * 2);
  auto copy_x_part = [&](char* t, int s, int c) __attribute__((always_inline)) {
    dma_lds16(rxw, t + (64 * p + 8 * c) * 128, vx + c * x_gstride, (uint32_t)(kfirst + s) * 128u);
  };
  auto copy_x = [&](char* t, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) copy_x_part(t, s, c);
  };
  // LoRA tiles (sT rows, B2 rows), the same pattern over rows of 2Rp bf16.
  const uint32_t vl = (uint32_t)(((64 * p + (lane >> 3)) * 2 * Rp + 8 * xlch) * 2);
  const uint32_t l_gstride = (uint32_t)(8 * 2 * Rp * 2);
  auto copy_lora = [&](rsrc_t r, char* t, int l) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      buf_load_lds16(r, t + (64 * p + 8 * c) * 128, vl, c * l_gstride + (uint32_t)l * 128u);
  };

  // Table of row 64p + lane for step t: the dword holding its e4m3 byte and
  // its group scale, loaded a step ahead; lane writes the 16 values
  // RNE_bf16(fl32(q_j * c')) (bit-identical to multiplying per element,
  // since the value depends only on code and row).
  const int trow = 64 * p + lane;
  const uint32_t ve_me = (uint32_t)trow * kpr;
  const uint32_t blk_me = (uint32_t)(n0 + trow) * kpr;
  struct Consts {
    uint32_t e, s;
  };
  auto load_consts = [&](Consts& r, int t) __attribute__((always_inline)) {
    r.e = buf_load4(re, (ve_me + (uint32_t)(kfirst + t)) & ~3u, 0u);
    r.s = buf_load4(rs, ((blk_me + (uint32_t)(kfirst + t)) / kDqBlock) * 4u, 0u);
  };
  const int tb_off = 32 * (lane & 7) + 256 * (8 * p + (lane >> 3));
  auto build_table = [&](int t, const Consts& r) __attribute__((always_inline)) {
    const uint32_t e = (r.e >> (8 * ((ve_me + (uint32_t)(kfirst + t)) & 3u))) & 0xffu;
    const float cp = decode_constant(e, __uint_as_float(r.s), mu);
    u32x4_t t0, t1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t0[j] = pack16<F16>(__fmul_rn(cb.q[2 * j], cp), __fmul_rn(cb.q[2 * j + 1], cp));
      t1[j] = pack16<F16>(__fmul_rn(cb.q[8 + 2 * j], cp), __fmul_rn(cb.q[9 + 2 * j], cp));
    }
    char* const d = stab[t & 1] + tb_off;
    *reinterpret_cast<u32x4_t*>(d) = t0;
    *reinterpret_cast<u32x4_t*>(d + 16) = t1;
  };

  const int PR0 = 128 + 32 * p;
  uint32_t cw[4], cwn[4];
  Consts cc, cn;
  // prologue: X of step 0, tables of steps 0 and 1, lookups of step 0
  {
    Consts c0;
    copy_x(sx0, 0);
    load_consts(c0, 0);
    load_consts(cn, 1);
    load_consts(cc, 2);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cw[q] = load_code(PR0 + 8 * q, 0);
      cwn[q] = load_code(PR0 + 8 * q, 1);
    }
    build_table(0, c0);
    build_table(1, cn);
  }
  __syncthreads();  // tables of steps 0 and 1 in place
  dequant_rows(std::integral_constant<int, 4>(), PR0, cw, 0, no_issue);
#pragma unroll
  for (int q = 0; q < 4; ++q) cw[q] = cwn[q];
  wait_vmem();
  __syncthreads();  // step 0 in place

  // Weight steps 0 .. ksteps-2: load the codes of step s+2 and constants of
  // step s+3, build the tables of step s+2 (that buffer was last read in the
  // previous iteration), dequantize this wave's rows of step s+1 while
  // copying X of step s+1 into the other X buffer.
#pragma unroll 1
  for (int s = 0; s + 1 < ksteps; ++s) {
    char* const xn = sxb((s + 1) & 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) cwn[q] = load_code(PR0 + 8 * q, s + 2);
    load_consts(cn, s + 3);
    build_table(s + 2, cc);
    dequant_rows(std::integral_constant<int, 4>(), PR0, cw, s + 1, [&](int q) {
      copy_x_part(xn, s + 1, 2 * q);
      copy_x_part(xn, s + 1, 2 * q + 1);
    });
#pragma unroll
    for (int q = 0; q < 4; ++q) cw[q] = cwn[q];
    cc = cn;
    wait_vmem();
    __syncthreads();
  }
  // last weight step: copy LoRA step 0 (sT and B2 tiles) into the other
  // buffers; then the LoRA steps
  if (lsteps > 0) {
    copy_lora(rt, sxb(ksteps & 1), 0);
    copy_lora(rb, sw[ksteps & 1], 0);
  }
  wait_vmem();
  __syncthreads();
#pragma unroll 1
  for (int l = 0; l < lsteps; ++l) {
    const int s = ksteps + l;
    if (l + 1 < lsteps) {
      copy_lora(rt, sxb((s + 1) & 1), l + 1);
      copy_lora(rb, sw[(s + 1) & 1], l + 1);
    }
    wait_vmem();
    __syncthreads();
  }
}

}  // namespace

int fwd_gemm_splits(int64_t M, int64_t N, int64_t K, size_t cap) {
  const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
  return gemm_splits(tiles, K / KSTEP, M, N, cap);
}

hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B2, int64_t Rp, void* Y, bool y16, int splits, float* P, bool f16,
                           hipStream_t st) {
  const int tm = (int)((M + TM - 1) / TM), tn = (int)((W.N + TN - 1) / TN);
  const unsigned grid = tile_grid(tm, tn, splits);
  const int yb = y16 ? 1 : 0;
  switch (2 * Rp / KSTEP) {
#define QNF4_FWD_CASE(LS)                                                                   \
  case LS:                                                                                  \
    return f16 ? timed_launch(kKernFwdGemm, fwd_gemm_kernel<LS, true>, dim3(grid), dim3(kThreads), st, W, X, M, \
                              (const uint16_t*)sT, (const uint16_t*)B2, Rp, Y, yb, tm, tn, splits, P, codebook()) \
               : timed_launch(kKernFwdGemm, fwd_gemm_kernel<LS, false>, dim3(grid), dim3(kThreads), st, W, X, M, \
                              (const uint16_t*)sT, (const uint16_t*)B2, Rp, Y, yb, tm, tn, splits, P, codebook());
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
