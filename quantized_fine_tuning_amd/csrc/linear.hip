// Host orchestration of the QLoRA linear layer (forward and backward): the
// order of the kernels, the workspace layout and the reduction slices.
//
// Forward (P1 §七 dataflow figure):  T = X·Aᵀ, Y = X·Ŵᵀ + s·T·Bᵀ.
// Backward (P1 简化版, P2 §4.4): U = dY·B, dX = dY·Ŵ + s·U·A,
// dA = s·Uᵀ·X, dB = s·dYᵀ·T; no gradient for the frozen weight.
// The low-rank factors T and U enter the big products as bf16 hi/lo splits
// of s·T and s·U (about 16 significant bits); dA and dB use the same splits.
#include <algorithm>

#include "host.h"

namespace qnf4 {

hipError_t launch_dx_gemm(const Nf4View& W, const uint16_t* dY, int64_t M, const uint16_t* sU,
                          const uint16_t* AT2, int64_t Rp, void* dX, bool dx16, int splits, float* P, bool f16,
                          hipStream_t st);
hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B2, int64_t Rp, void* Y, bool y16, int splits, float* P, bool f16,
                           hipStream_t st);
hipError_t launch_splitk_reduce(const float* P, int splits, int64_t n, void* out, bool out16, bool f16,
                                hipStream_t st);
int fwd_gemm_splits(int64_t M, int64_t N, int64_t K, size_t cap);
int dx_gemm_splits(int64_t M, int64_t N, int64_t K, size_t cap);
hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                       int32_t r, float scale, void* Y, bool y16, float* T, float* P, bool f16, hipStream_t st);

FwdLayout fwd_layout(int64_t M, int64_t N, int64_t K, int32_t r, size_t cap) {
  FwdLayout L{};
  L.splits = 1;
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
    L.pT = rowred_plan(M, K, Rp);
    const size_t p = round_up(rowred_partial_bytes(L.pT), 256);
    L.splits = fwd_gemm_splits(M, N, K, cap > off ? cap - off : 0);
    off += L.splits > 1 ? std::max<size_t>(p, round_up((size_t)L.splits * M * N * 4, 256)) : p;
  } else if (M > 0) {
    off += round_up(gemv_partial_bytes(K, r), 256);  // partial tiles of T
  }
  L.total = off;
  return L;
}

BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int32_t r) {
  BwdLayout L{};
  const int64_t Rp = lora_rp(r), Mp = lora_mp(M);
  if (M > 0) {
    L.pT = rowred_plan(M, K, Rp);
    L.pU = rowred_plan(M, N, Rp);
    const uint32_t ga = colred_split(K, N, Rp);
    L.pA = colred_plan(M, K, Rp, ga);
    L.pB = colred_plan(M, N, Rp, kSkWorkgroups - ga);
  }
  size_t off = 0;
  L.off_sT = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_sTT = off;
  off += round_up(2 * Rp * Mp * 2, 256);
  L.off_sU = off;
  off += round_up(M * 2 * Rp * 2, 256);
  L.off_sUT = off;
  off += round_up(2 * Rp * Mp * 2, 256);
  L.off_BT = off;
  off += round_up(Rp * round_up(N, 64) * 2, 256);
  L.off_AT2 = off;
  off += round_up(K * 2 * Rp * 2, 256);
  // one partial-sum area reused by the successive reductions
  L.off_P = off;
  size_t p = 0;
  L.splits = 1;
  if (M > 0) {
    p = std::max<size_t>(p, round_up(rowred_partial_bytes(L.pT), 256));
    p = std::max<size_t>(p, round_up(rowred_partial_bytes(L.pU), 256));
    // dA's and dB's partial tiles side by side (one launch)
    p = std::max<size_t>(p, round_up(colred_partial_bytes(L.pA), 256) + round_up(colred_partial_bytes(L.pB), 256));
    L.splits = dx_gemm_splits(M, N, K, SIZE_MAX);
    if (L.splits > 1) p = std::max<size_t>(p, round_up((size_t)L.splits * M * K * 4, 256));
  }
  off += p;
  L.total = off;
  return L;
}

// Workspace bytes that cover every M in [0, M_max].  The split reductions'
// partial-sum areas (tiles x cmax slots) are not monotone in M: cmax, the
// most workgroups that share one tile, depends on how the tiles fall on the
// workgroups.  Every plan depends on M only through ceil(M / 64), so the
// maximum is taken over those values; where a plan has at least as many
// tiles as workgroups, each workgroup's run covers a whole tile's units and
// cmax <= 2, so tiles x 2 slots bound it (monotone in M) and the exact plan
// is not needed there.
namespace {
size_t rowred_bytes_bound(int64_t M, int64_t Kred, int64_t Rp) {
  const int64_t tiles = ((M + 63) / 64) * ((Rp + 63) / 64);
  if (tiles >= (int64_t)kSkWorkgroups) return round_up(tiles * 2 * 64 * 64 * 4, 256);
  return round_up(rowred_partial_bytes(rowred_plan(M, Kred, Rp)), 256);
}
size_t colred_bytes_bound(int64_t M, int64_t Pn, int64_t Rp, uint32_t gmax) {
  const int64_t tiles = ((Pn + 127) / 128) * ((Rp + 63) / 64);
  if (tiles >= (int64_t)gmax) return round_up(tiles * 2 * 128 * 64 * 4, 256);
  return round_up(colred_partial_bytes(colred_plan(M, Pn, Rp, gmax)), 256);
}
// The GEMMs' split partials over M in [1, M_max] (the forward GEMM runs
// from 17 tokens on, the dX GEMM from 1): the split count depends on M only
// through the number of 256-row tiles, and within one such band the bytes
// grow with M, so each band's largest M is taken.
size_t splitk_bytes_max(int64_t M_max, int64_t N, int64_t K, bool fwd) {
  size_t p = 0;
  for (int64_t top = 256;; top += 256) {
    const int64_t M = std::min(top, M_max);
    if (M > (fwd ? 16 : 0)) {
      const int s = fwd ? fwd_gemm_splits(M, N, K, SIZE_MAX) : dx_gemm_splits(M, N, K, SIZE_MAX);
      if (s > 1) p = std::max<size_t>(p, round_up((size_t)s * M * (fwd ? N : K) * 4, 256));
    }
    if (top >= M_max) break;
  }
  return p;
}
}  // namespace

size_t fwd_ws_bytes_max(int64_t M_max, int64_t N, int64_t K, int32_t r) {
  // M <= 16 (the GEMV path) grows with M; M > 16 is the GEMM path
  const size_t small = fwd_layout(std::min<int64_t>(M_max, 16), N, K, r).total;
  if (M_max <= 16) return small;
  const FwdLayout L = fwd_layout(M_max, N, K, r);
  const int64_t Rp = lora_rp(r);
  size_t p = splitk_bytes_max(M_max, N, K, true);
  for (int64_t M = 64; M < M_max + 64; M += 64) p = std::max(p, rowred_bytes_bound(std::min(M, M_max), K, Rp));
  return std::max(small, L.off_P + p);
}

size_t bwd_ws_bytes_max(int64_t M_max, int64_t N, int64_t K, int32_t r) {
  const BwdLayout L = bwd_layout(M_max, N, K, r);
  if (M_max <= 0) return L.total;
  const int64_t Rp = lora_rp(r);
  const uint32_t ga = colred_split(K, N, Rp);
  size_t p = splitk_bytes_max(M_max, N, K, false);
  for (int64_t M = 64; M < M_max + 64; M += 64) {
    const int64_t m = std::min(M, M_max);
    p = std::max({p, rowred_bytes_bound(m, K, Rp), rowred_bytes_bound(m, N, Rp),
                  colred_bytes_bound(m, K, Rp, ga) + colred_bytes_bound(m, N, Rp, kSkWorkgroups - ga)});
  }
  return L.off_P + p;
}

hipError_t launch_forward(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                          const uint16_t* B, int32_t r, float scale, void* Y, bool y16,
                          float* T, char* ws, const FwdLayout& L, bool f16, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (M <= 16)
    return launch_gemv(W, X, M, A, B, r, scale, Y, y16, T, reinterpret_cast<float*>(ws + L.off_P), f16, st);
  const int64_t Rp = lora_rp(r);
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  float* P = reinterpret_cast<float*>(ws + L.off_P);
  hipError_t e = launch_rowred(X, M, W.K, W.K, A, r, W.K, L.pT, P, f16, st);
  if (e != hipSuccess) return e;
  uint16_t* B2 = reinterpret_cast<uint16_t*>(ws + L.off_B2);
  e = launch_rowred_finish(P, L.pT, M, r, Rp, scale, T, sT, nullptr, B, W.N, B2, f16, st);
  if (e != hipSuccess) return e;
  // (the partial sums of T have been consumed: P now takes the split partials)
  e = launch_fwd_gemm(W, X, M, sT, B2, Rp, Y, y16, L.splits, P, f16, st);
  if (e != hipSuccess || L.splits == 1) return e;
  return launch_splitk_reduce(P, L.splits, M * W.N, Y, y16, f16, st);
}

hipError_t launch_backward(const Nf4View& W, const uint16_t* X, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                           const float* T_saved, void* dX, bool dx16, float* dA, float* dB,
                           char* ws, const BwdLayout& L, bool f16, hipStream_t st) {
  const int64_t Rp = lora_rp(r), Mp = lora_mp(M);
  const int64_t N = W.N, K = W.K;
  float* P = reinterpret_cast<float*>(ws + L.off_P);
  hipError_t e;
  if (M == 0) {  // no tokens: the adapter gradients are zero
    e = launch_zero(dA, (int64_t)r * K, st);
    if (e != hipSuccess) return e;
    return launch_zero(dB, N * r, st);
  }
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  uint16_t* sTT = reinterpret_cast<uint16_t*>(ws + L.off_sTT);
  uint16_t* sU = reinterpret_cast<uint16_t*>(ws + L.off_sU);
  uint16_t* sUT = reinterpret_cast<uint16_t*>(ws + L.off_sUT);
  uint16_t* BT = reinterpret_cast<uint16_t*>(ws + L.off_BT);
  uint16_t* AT2 = reinterpret_cast<uint16_t*>(ws + L.off_AT2);
  // operand copies: s·T (hi/lo and transposed) from the saved T, Bᵀ, [Aᵀ | Aᵀ]
  e = launch_bwd_prep(T_saved, M, r, Rp, scale, sT, sTT, B, N, BT, A, K, AT2, f16, st);
  if (e != hipSuccess) return e;
  if (!T_saved) {  // s·T recomputed
    e = launch_rowred(X, M, K, K, A, r, K, L.pT, P, f16, st);
    if (e == hipSuccess)
      e = launch_rowred_finish(P, L.pT, M, r, Rp, scale, nullptr, sT, sTT, nullptr, 0, nullptr, f16, st);
    if (e != hipSuccess) return e;
  }
  // s·U, U = dY·B
  e = launch_rowred(dY, M, N, N, BT, Rp, round_up(N, 64), L.pU, P, f16, st);
  if (e == hipSuccess) e = launch_rowred_finish(P, L.pU, M, r, Rp, scale, nullptr, sU, sUT, nullptr, 0, nullptr, f16, st);
  if (e != hipSuccess) return e;
  // dX = [dY | sU_hi | sU_lo] · [Ŵ ; A ; A]
  e = launch_dx_gemm(W, dY, M, sU, AT2, Rp, dX, dx16, L.splits, P, f16, st);
  if (e == hipSuccess && L.splits > 1) e = launch_splitk_reduce(P, L.splits, M * K, dX, dx16, f16, st);
  if (e != hipSuccess) return e;
  // dA[j][k] = Σ_m (sU_hi + sU_lo)[m][j] · X[m][k]   (s is inside sU) and
  // dB[n][j] = Σ_m dY[m][n] · (sT_hi + sT_lo)[m][j], in one launch, their
  // partial tiles side by side
  float* PB = P + round_up(colred_partial_bytes(L.pA), 256) / 4;
  const ColredJob ja{X, M, K, sUT, Mp, Rp, L.pA.jt, L.pA.ut, L.pA.U, L.pA.G, L.pA.cmax, P};
  const ColredJob jb{dY, M, N, sTT, Mp, Rp, L.pB.jt, L.pB.ut, L.pB.U, L.pB.G, L.pB.cmax, PB};
  e = launch_colred(ja, jb, f16, st);
  if (e != hipSuccess) return e;
  const ColredFinishJob fa{P, L.pA.jt, L.pA.ut, L.pA.U, L.pA.G, L.pA.cmax, K, L.pA.tiles, 1, dA};
  const ColredFinishJob fb{PB, L.pB.jt, L.pB.ut, L.pB.U, L.pB.G, L.pB.cmax, N, L.pB.tiles, 0, dB};
  return launch_colred_finish(fa, fb, r, st);
}

}  // namespace qnf4
