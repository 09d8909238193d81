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
                          const uint16_t* AT2, int64_t Rp, void* dX, bool dx16, bool f16, hipStream_t st);
hipError_t launch_fwd_gemm(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* sT,
                           const uint16_t* B2, int64_t Rp, void* Y, bool y16, bool f16, hipStream_t st);
hipError_t launch_gemv(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                       const uint16_t* B, int32_t r, float scale, void* Y, bool y16, float* T,
                       bool f16, hipStream_t st);

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
    L.pT = rowred_plan(M, K, Rp);
    off += round_up(rowred_partial_bytes(L.pT), 256);
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
    L.pA = colred_plan(M, K, Rp);
    L.pB = colred_plan(M, N, Rp);
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
  if (M > 0) {
    p = std::max<size_t>(p, round_up(rowred_partial_bytes(L.pT), 256));
    p = std::max<size_t>(p, round_up(rowred_partial_bytes(L.pU), 256));
    p = std::max<size_t>(p, round_up(colred_partial_bytes(L.pA), 256));
    p = std::max<size_t>(p, round_up(colred_partial_bytes(L.pB), 256));
  }
  off += p;
  L.total = off;
  return L;
}

hipError_t launch_forward(const Nf4View& W, const uint16_t* X, int64_t M, const uint16_t* A,
                          const uint16_t* B, int32_t r, float scale, void* Y, bool y16,
                          float* T, char* ws, const FwdLayout& L, bool f16, hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (M <= 16) {
    float* Tw = T ? T : reinterpret_cast<float*>(ws + L.off_T);
    return launch_gemv(W, X, M, A, B, r, scale, Y, y16, Tw, f16, st);
  }
  const int64_t Rp = lora_rp(r);
  uint16_t* sT = reinterpret_cast<uint16_t*>(ws + L.off_sT);
  float* P = reinterpret_cast<float*>(ws + L.off_P);
  hipError_t e = launch_rowred(X, M, W.K, W.K, A, r, W.K, L.pT, P, f16, st);
  if (e != hipSuccess) return e;
  uint16_t* B2 = reinterpret_cast<uint16_t*>(ws + L.off_B2);
  e = launch_rowred_finish(P, L.pT, M, r, Rp, scale, T, sT, nullptr, B, W.N, B2, f16, st);
  if (e != hipSuccess) return e;
  return launch_fwd_gemm(W, X, M, sT, B2, Rp, Y, y16, f16, st);
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
  e = launch_dx_gemm(W, dY, M, sU, AT2, Rp, dX, dx16, f16, st);
  if (e != hipSuccess) return e;
  // dA[j][k] = Σ_m (sU_hi + sU_lo)[m][j] · X[m][k]   (s is inside sU)
  e = launch_colred(X, M, K, K, sUT, Mp, Rp, L.pA, P, f16, st);
  if (e == hipSuccess) e = launch_colred_finish(P, L.pA, K, r, true, dA, st);
  if (e != hipSuccess) return e;
  // dB[n][j] = Σ_m dY[m][n] · (sT_hi + sT_lo)[m][j]
  e = launch_colred(dY, M, N, N, sTT, Mp, Rp, L.pB, P, f16, st);
  if (e == hipSuccess) e = launch_colred_finish(P, L.pB, N, r, false, dB, st);
  return e;
}

}  // namespace qnf4
