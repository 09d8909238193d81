// Forward product of the QLoRA linear layer for M > 16 tokens, gfx950:
//   Y[M, N] = X·Ŵᵀ + s·T·Bᵀ  =  [X | sT_hi | sT_lo] · [Ŵ | B | B]ᵀ
// (P1 §七 dataflow figure: the 4-bit base is dequantized to BF16 for the
// matmul and the LoRA path is added to the output.)
//
// Design
//   * One output tile per workgroup of 12 waves, three per SIMD, in two
//     roles; the tile is 256x256, or 512x128 from 2048 tokens on and from
//     512 on where it adds no padding rows (one kernel template, TMV = 256 or
//     512 token rows).  Waves 0..7 only
//     multiply: wave (wm, wn) owns token rows [128wm, +128) and weight rows
//     [64wn, +64) of the tile (2 x 4 waves, or 4 x 2), 64
//     v_mfma_f32_16x16x32_bf16 per 64-wide reduction step, operands read
//     from LDS one MFMA group ahead.  Waves 8..11 (one per SIMD) produce the
//     operands of the next step: each copies a quarter of the X tile
//     straight into LDS and dequantizes a quarter of the tile's weight rows
//     into the shared bf16 tile Ŵ[n][k].  Their arithmetic and copies
//     overlap the MFMAs of the other two waves of their SIMD.
//   * The 512x128 tile decodes each weight row of a step once for 512
//     tokens: half the producers' decode per MFMA for twice their X copy
//     (64 KB of X and 16 KB of Ŵ per step, 160 KB of LDS with both
//     buffers).  On the 7B MLP shapes it takes the forward GEMM from ≈322 to
//     ≈310 µs (bit-identical output), at 1,024–1,536 tokens by 4-6 % (with
//     or without a split reduction).
//   * Dequantization in registers: producer p owns tile rows
//     [WR p, +WR) (WR = 64 or 32): lane l takes row WR p + l % WR and, when
//     two lanes share a row, half l / WR of its 64 codes.  Per step a lane
//     builds its row's table of the 16 values RNE_bf16(fl32(q_j * c')) of
//     the step's block (bit-identical to multiplying per element, since the
//     value depends only on code and row), held as four byte planes (low
//     bytes of values 0-3, 4-7, 8-11, 12-15, likewise the high bytes), and
//     decodes its codes with byte permutes: four codes per permute pair,
//     the code's low three bits selecting within 8 bytes and its top bit
//     between the two halves; the low and high bytes are then interleaved
//     into bf16 pairs and the row's 16-byte chunks stored.  No LDS lookups,
//     no tables in LDS.
//   * Each producer step first waits for the codes and constants it loaded a
//     step earlier, then issues the X copy of the next step, then the loads
//     of the step after (into the other of two register sets, so that no
//     register a load in flight writes is copied), then decodes; at its end
//     only the X copy must be complete.  (The X copy is the long-latency
//     transfer; issued first it has the whole step to land.)
//   * Tiles are stored with 16-byte chunks XOR-swizzled by row (xswz) so that
//     MFMA operand reads of 8 rows cover the 32 LDS banks once.
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

constexpr int TM = 256, TN = 256, KSTEP = 64;  // the square tile (split plans)
constexpr int kMfmaWaves = 8, kProdWaves = 4, kWaves = kMfmaWaves + kProdWaves;
constexpr int kThreads = 64 * kWaves;
// 512 x 128 tiles from 2048 tokens on, and from 512 tokens on where they
// add no padding rows over 256-row tiles
constexpr int64_t kTallMinTokens = 512, kTallAlwaysTokens = 2048;
inline bool fwd_tall(int64_t M) {
  return M >= kTallAlwaysTokens || (M >= kTallMinTokens && ((M + 255) / 256) % 2 == 0);
}

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

// TMV x (65536 / TMV) output tiles: 256 x 256, or 512 x 128 (the weight
// rows of a step decoded once for twice the tokens: half the producers'
// decode per MFMA, twice their X copy).
template <int LSTEPS, bool F16, int TMV>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(Nf4View W, const uint16_t* __restrict__ X,
                                                               int64_t M, const uint16_t* __restrict__ sT,
                                                               const uint16_t* __restrict__ B2,
                                                               int64_t Rp, void* __restrict__ Y,
                                                               int y_bf16, int tiles_m, int tiles_n,
                                                               int splits, float* __restrict__ P,
                                                               Codebook cb) {
  constexpr int TM = TMV, TN = 65536 / TMV;
  constexpr int WGN = TN / 64;           // MFMA waves along N (4 or 2), each 128 x 64
  constexpr int XR = TM / kProdWaves;    // X rows copied per producer and step (64 or 128)
  constexpr int WR = TN / kProdWaves;    // weight rows decoded per producer (64 or 32)
  constexpr int HALVES = 64 / WR;        // lanes per weight row (1 or 2)
  constexpr int NLOADS = 2 / HALVES + 2;  // vector loads per producer step (codes, e byte, scale)
  __shared__ __attribute__((aligned(16))) char sx0[TM * 128], sx1[TM * 128];  // A tiles: X, then sT
  __shared__ __attribute__((aligned(16))) char sw[2][TN * 128];  // B tiles: Ŵ, then B2
  int tmi, tni, sp;
  if (!tile_of<TMV == 512 ? 2 : kGroupM>(blockIdx.x, tiles_m, tiles_n, splits, tmi, tni, sp)) return;

  // (the wave index in a scalar register: the LDS addresses and offsets of
  // the copies derived from it are then formed by scalar instructions)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  auto no_issue = [](int) {};

  if (wave < kMfmaWaves) {
    // ---------------------------------------------------------------- MFMA
    const int lr = lane & 15, kq = lane >> 4;
    const int wm = wave / WGN, wn = wave % WGN;
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // MFMA group g (0..15) of a step: k-half ks = g / 8, token block i = g % 8.
    // A fragments are read one group ahead: group g first reads the A
    // fragment of group g + 1, so the read's latency overlaps this group's
    // MFMAs.  At a step's start the A fragment of group 0 is requested before
    // the four B fragments, so that its first MFMA waits for two reads, not
    // five (LDS reads return in order; about 1% on the step).  The B
    // fragments of the second k-half are read right after the MFMAs of
    // group 7.
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
      anext = read_a(xa, 0);
      read_b(wb, 0, bfr);
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

    __syncthreads();  // (the producers' prologue)
    __syncthreads();  // step 0 in place
#pragma unroll 1
    for (int s = 0; s + 1 < ksteps; ++s) {
      mfma_step(sxb(s & 1), sw[s & 1]);
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
  // Producer p dequantizes weight rows [WR p, +WR) and copies X rows
  // [XR p, +XR) of every step (WR = XR = 64 on the square tile; WR = 32,
  // XR = 128 on the tall one).
  const int p = wave - kMfmaWaves;
  const uint32_t kpr = (uint32_t)(K / kBlock);  // blocks per weight row
  const float mu = *W.mu;
  const rsrc_t rt = make_rsrc(sT + m0 * 2 * Rp, (M - m0) * 2 * Rp * 2);
  const rsrc_t re = make_rsrc(W.e + n0 * kpr, (N - n0) * kpr);
  const rsrc_t rs = make_rsrc(W.s, ((N * kpr + kDqBlock - 1) / kDqBlock) * 4);
  const rsrc_t rb = make_rsrc(B2 + n0 * 2 * Rp, (N - n0) * 2 * Rp * 2);

  // X rows [XR p, +XR) of a step, copied straight into LDS: part c
  // moves rows XR p + 8c + (l >> 3), lane l into physical chunk l & 7, so it
  // fetches logical chunk (l & 7) ^ sw(l >> 3) (row & 7 = l >> 3).  Each
  // instruction fills 1 KB of LDS contiguously.  (Written as assembly: the
  // compiler then inserts no wait for these copies in front of the
  // producer's own LDS reads; the wait before the step's closing barrier is
  // explicit.)
  const int xlch = (lane & 7) ^ rsw(lane >> 3);
  const uint32_t vx = (uint32_t)(((XR * p + (lane >> 3)) * K + 8 * xlch) * 2);
  const uint32_t x_gstride = (uint32_t)(8 * K * 2);
  const i32x4_t rxw = rsrc_words(X + m0 * K, (M - m0) * K * 2);
  auto copy_x_part = [&](char* t, int s, int c) __attribute__((always_inline)) {
    dma_lds16(rxw, t + (XR * p + 8 * c) * 128, vx + c * x_gstride, (uint32_t)(kfirst + s) * 128u);
  };
  auto copy_x = [&](char* t, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < XR / 8; ++c) copy_x_part(t, s, c);
  };
  // LoRA tiles (sT rows, B2 rows), the same pattern over rows of 2Rp bf16.
  const uint32_t l_gstride = (uint32_t)(8 * 2 * Rp * 2);
  auto copy_lora = [&](rsrc_t r, char* t, int l, auto rows) __attribute__((always_inline)) {
    constexpr int RR = decltype(rows)::value;  // rows per producer
    const uint32_t vl = (uint32_t)(((RR * p + (lane >> 3)) * 2 * Rp + 8 * xlch) * 2);
#pragma unroll
    for (int c = 0; c < RR / 8; ++c)
      buf_load_lds16(r, t + (RR * p + 8 * c) * 128, vl, c * l_gstride + (uint32_t)l * 128u);
  };
  using XRows = std::integral_constant<int, XR>;
  using WRows = std::integral_constant<int, WR>;

  // Row trow = WR p + lane % WR of the tile is this lane's: the dword
  // holding its e4m3 byte and its group scale, and per step its 32 bytes of
  // codes (the 16 of half lane / WR when two lanes share the row).
  const int trow = WR * p + lane % WR, half = lane / WR;
  const uint32_t ve_me = (uint32_t)trow * kpr;
  const uint32_t blk_me = (uint32_t)(n0 + trow) * kpr;
  struct Consts {
    uint32_t e, s;
  };
  auto load_consts = [&](Consts& r, int t) __attribute__((always_inline)) {
    r.e = buf_load4(re, (ve_me + (uint32_t)(kfirst + t)) & ~3u, 0u);
    r.s = buf_load4(rs, ((blk_me + (uint32_t)(kfirst + t)) / kDqBlock) * 4u, 0u);
  };
  const uint32_t vrow = (uint32_t)trow * (uint32_t)(K / 2);
  auto load_row = [&](u32x4_t* c, int t) __attribute__((always_inline)) {
    if constexpr (HALVES == 1) {
      c[0] = buf_load16(rc, vrow, (uint32_t)(kfirst + t) * 32u);
      c[1] = buf_load16(rc, vrow, (uint32_t)(kfirst + t) * 32u + 16u);
    } else {
      c[0] = buf_load16(rc, vrow + 16u * (uint32_t)half, (uint32_t)(kfirst + t) * 32u);
    }
  };
  auto row_table = [&](int t, const Consts& r, uint32_t* L, uint32_t* H) __attribute__((always_inline)) {
    const uint32_t e = (r.e >> (8 * ((ve_me + (uint32_t)(kfirst + t)) & 3u))) & 0xffu;
    const float cp = decode_constant(e, __uint_as_float(r.s), mu);
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = pack16<F16>(__fmul_rn(cb.q[2 * j], cp), __fmul_rn(cb.q[2 * j + 1], cp));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      L[g] = __builtin_amdgcn_perm(d[2 * g + 1], d[2 * g], 0x06040200u);
      H[g] = __builtin_amdgcn_perm(d[2 * g + 1], d[2 * g], 0x07050301u);
    }
  };
  // T: a byte plane; the bytes of c are four codes (0..15)
  auto look = [&](uint32_t c, const uint32_t* T) __attribute__((always_inline)) {
    const uint32_t s7 = c & 0x07070707u;
    const uint32_t sel = ((c >> 1) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(__builtin_amdgcn_perm(T[3], T[2], s7), __builtin_amdgcn_perm(T[1], T[0], s7), sel);
  };
  // eight codes (one dword: element 2b in the low nibble of byte b, 2b+1 in
  // its high nibble) into four bf16 pairs in element order
  auto decode8 = [&](uint32_t w, const uint32_t* L, const uint32_t* H, u32x4_t& o) __attribute__((always_inline)) {
    const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t le = look(ev, L), he = look(ev, H), lo = look(od, L), ho = look(od, H);
    const uint32_t E01 = __builtin_amdgcn_perm(he, le, 0x05010400u), E23 = __builtin_amdgcn_perm(he, le, 0x07030602u);
    const uint32_t O01 = __builtin_amdgcn_perm(ho, lo, 0x05010400u), O23 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);
    o[0] = __builtin_amdgcn_perm(O01, E01, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(O01, E01, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(O23, E23, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(O23, E23, 0x07060302u);
  };
  auto decode_row = [&](const u32x4_t* c, const uint32_t* L, const uint32_t* H, char* dst, auto&& issue)
      __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 8 / HALVES; ++jj) {
      const int j = HALVES == 1 ? jj : 4 * half + jj;  // chunk of the row
      u32x4_t o;
      decode8(c[jj >> 2][jj & 3], L, H, o);
      *reinterpret_cast<u32x4_t*>(dst + xswz(trow, j)) = o;
      issue(jj);
    }
  };

  u32x4_t cw[2], cwn[2];
  Consts cc, cn;
  // prologue: X of step 0, codes and constants of steps 0 and 1, step 0 decoded
  {
    Consts c0;
    u32x4_t k0[2];
    copy_x(sx0, 0);
    load_consts(c0, 0);
    load_consts(cc, 1);
    load_row(k0, 0);
    load_row(cw, 1);
    uint32_t L[4], H[4];
    row_table(0, c0, L, H);
    decode_row(k0, L, H, sw[0], no_issue);
  }
  __syncthreads();
  wait_vmem();
  __syncthreads();  // step 0 in place

  // Weight steps 0 .. ksteps-2, one step: the table of step s+1 from constants loaded a step earlier
  // (their first use, where the compiler waits for them), then the X copy of
  // step s+1 and the loads of step s+2 (into the other register set: no
  // copies of registers that loads in flight are writing), then the decode;
  // at the end the X copy must be done while the 4 loads of step s+2 may
  // still be in flight.
  auto pstep = [&](int s, const u32x4_t* cur, u32x4_t* nxt, const Consts& ccur, Consts& cnxt)
      __attribute__((always_inline)) {
    uint32_t L[4], H[4];
    row_table(s + 1, ccur, L, H);
    // the table and this step's codes exist before the copies are issued
    // (the compiler's waits for them would otherwise also wait for copies
    // issued before them, which it does not track)
    asm volatile("" : "+v"(L[0]), "+v"(L[1]), "+v"(L[2]), "+v"(L[3]), "+v"(H[0]), "+v"(H[1]), "+v"(H[2]),
                 "+v"(H[3]) : "v"(cur[0]), "v"(cur[HALVES == 1 ? 1 : 0]));
    copy_x(sxb((s + 1) & 1), s + 1);
    load_row(nxt, s + 2);
    load_consts(cnxt, s + 2);
    decode_row(cur, L, H, sw[(s + 1) & 1], no_issue);
    wait_vmem_le<NLOADS>();
    __syncthreads();
  };
#pragma unroll 1
  for (int s = 0; s + 1 < ksteps; s += 2) {
    pstep(s, cw, cwn, cc, cn);
    if (s + 2 < ksteps) pstep(s + 1, cwn, cw, cn, cc);
  }
  // last weight step: copy LoRA step 0 (sT and B2 tiles) into the other
  // buffers; then the LoRA steps
  if (lsteps > 0) {
    copy_lora(rt, sxb(ksteps & 1), 0, XRows{});
    copy_lora(rb, sw[ksteps & 1], 0, WRows{});
  }
  wait_vmem();
  __syncthreads();
#pragma unroll 1
  for (int l = 0; l < lsteps; ++l) {
    const int s = ksteps + l;
    if (l + 1 < lsteps) {
      copy_lora(rt, sxb((s + 1) & 1), l + 1, XRows{});
      copy_lora(rb, sw[(s + 1) & 1], l + 1, WRows{});
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
  // 512 x 128 tiles (also with a split reduction: the split ranges, and so
  // every output's order of additions, are those of the square tile)
  const bool tall = fwd_tall(M);
  const int tmv = tall ? 512 : 256;
  const int tm = (int)((M + tmv - 1) / tmv), tn = (int)((W.N + 65536 / tmv - 1) / (65536 / tmv));
  const unsigned grid = tile_grid(tm, tn, splits);
  const int yb = y16 ? 1 : 0;
#define QNF4_FWD_LAUNCH(LS, F16V, TMV)                                                                        \
  timed_launch(kKernFwdGemm, fwd_gemm_kernel<LS, F16V, TMV>, dim3(grid), dim3(kThreads), st, W, X, M,        \
               (const uint16_t*)sT, (const uint16_t*)B2, Rp, Y, yb, tm, tn, splits, P, codebook())
#define QNF4_FWD_CASE(LS)                                                                                    \
  case LS:                                                                                                   \
    if (tall) return f16 ? QNF4_FWD_LAUNCH(LS, true, 512) : QNF4_FWD_LAUNCH(LS, false, 512);                 \
    return f16 ? QNF4_FWD_LAUNCH(LS, true, 256) : QNF4_FWD_LAUNCH(LS, false, 256);
  switch (2 * Rp / KSTEP) {
    QNF4_FWD_CASE(1)
    QNF4_FWD_CASE(2)
    QNF4_FWD_CASE(3)
    QNF4_FWD_CASE(4)
    QNF4_FWD_CASE(5)
    QNF4_FWD_CASE(6)
    QNF4_FWD_CASE(7)
    QNF4_FWD_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QNF4_FWD_CASE
#undef QNF4_FWD_LAUNCH
}

}  // namespace qnf4
