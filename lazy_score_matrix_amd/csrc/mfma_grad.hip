// Matrix-core backward of dot-product scores (float32): the gradients of
// softmax(S)@V and of the row log-sum-exp of S = r_i (X Y^T) + p_i by replay
// (torchpairwise guide: backward re-evaluates the pairs), as FlashAttention-2
// arranges it: nothing of size N x M is stored.
//
// Row side (a workgroup owns 128 rows i, key tiles stream through LDS):
//   S^T block   K . (r_i log2e X_i)^T               (matrix cores)
//   dP^T block  V . G_i^T                          (softmax; matrix cores)
//   P           2^(S - c_i),  c_i = (lse_i - p_i) log2e
//   dS          P (dP - delta_i)   or   g_i P     (logsumexp)
//   dX_i        r_i sum_j dS_ij y_j                 (matrix cores, K as operand)
// Column side (a workgroup owns 128 columns j, row tiles stream):
//   S^T block   (r_i X_i) . Y_j^T, dP^T block G_i . V_j^T
//   dV_j        sum_i P_ij G_i,  dY_j = sum_i dS_ij r_i x_i
// Both use the forward engine's layout: lane l owns the row (column) l % 32
// and holds 16 scores of the streamed side per 32-wide sub-block, so the same
// registers are the B operand of the second contraction. Column splits give
// partial sums that the shared merge kernel adds in split order.
#include "mfma_engine.h"

namespace pw {
namespace {

constexpr int kGWaves = 4, kGThreads = 256, kGBN = 64;

template <int CONS, int DP, int CP, int SIDE>
__global__ __launch_bounds__(kGThreads, 2) void mfma_grad_kernel(const MfmaGradArgs a) {
  using F = Mfma<float>;
  using acc_t = F::acc_t;
  constexpr int TM = 32, G = 2, NREG = 16, BN = kGBN, SB = BN / TM;
  constexpr bool SMX = CONS == C_SOFTMAX;
  constexpr int DG = DP / G, CG = CP / G;
  constexpr int ND = (DP + TM - 1) / TM, NC = CP / TM;
  constexpr int KP = 4;
  constexpr int CPS = SMX ? CP : 4;
  constexpr float L2E = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) float sA[BN][DP + KP];   // Y_j (row side), r_i X_i (column side)
  __shared__ __attribute__((aligned(16))) float sB[BN][CPS + KP];  // V_j (row side), G_i (column side)
  __shared__ float sC[BN], sD[BN];                                  // column side: c_i, delta_i or g_i

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, q = l & 31;
  const int rb = blockIdx.x % a.n_rb, sp = blockIdx.x / a.n_rb;
  const int64_t n_own = SIDE == 0 ? a.N : a.M, n_oth = SIDE == 0 ? a.M : a.N;
  const int64_t o = (int64_t)rb * (kGWaves * TM) + w * TM + q;
  const bool ov = o < n_own;
  const int64_t qb = (int64_t)sp * a.split, qe = min(n_oth, qb + a.split);

  // ---- own operands
  float pa[DG], pb[SMX ? CG : 1];
  float ci = 0, di = 0, ri = 1;
  if (SIDE == 0) {
    float r = a.r_s, p = a.p_s;
    if (a.row_vec && ov) {
      r = a.r_vec[o];
      p = a.p_vec[o];
    }
    ri = r;
    if (ov) {
      ci = (a.lse[o] - p) * L2E;
      di = SMX ? a.delta[o] : a.G[o * a.ldg];
    }
#pragma unroll
    for (int st = 0; st < DG; ++st) {
      const int d = g * DG + st;
      pa[st] = (ov && d < a.D) ? a.X[o * a.ldx + d] * (r * L2E) : 0.f;
    }
    if constexpr (SMX) {
#pragma unroll
      for (int st = 0; st < CG; ++st) {
        const int c = g * CG + st;
        pb[st] = (ov && c < a.C) ? a.G[o * a.ldg + c] : 0.f;
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < DG; ++st) {
      const int d = g * DG + st;
      pa[st] = (ov && d < a.D) ? a.Y[o * a.ldy + d] : 0.f;
    }
    if constexpr (SMX) {
#pragma unroll
      for (int st = 0; st < CG; ++st) {
        const int c = g * CG + st;
        pb[st] = (ov && c < a.C) ? a.V[o * a.ldv + c] : 0.f;
      }
    }
  }
  acc_t oa[ND], ob[SMX && SIDE == 1 ? NC : 1];
#pragma unroll
  for (int c = 0; c < ND; ++c)
#pragma unroll
    for (int r = 0; r < NREG; ++r) oa[c][r] = 0;
#pragma unroll
  for (int c = 0; c < (SMX && SIDE == 1 ? NC : 1); ++c)
#pragma unroll
    for (int r = 0; r < NREG; ++r) ob[c][r] = 0;

  for (int64_t q0 = qb; q0 < qe; q0 += BN) {
    const int nb = (int)min((int64_t)BN, qe - q0);
    __syncthreads();
    for (int e = tid; e < BN * DP; e += kGThreads) {
      const int jj = e / DP, d = e % DP;
      float v = 0;
      if (jj < nb && d < a.D) {
        const int64_t t = q0 + jj;
        if (SIDE == 0) v = a.Y[t * a.ldy + d];
        else v = a.X[t * a.ldx + d] * (a.row_vec ? a.r_vec[t] : a.r_s);
      }
      sA[jj][d] = v;
    }
    if constexpr (SMX) {
      for (int e = tid; e < BN * CP; e += kGThreads) {
        const int jj = e / CP, c = e % CP;
        float v = 0;
        if (jj < nb && c < a.C) v = SIDE == 0 ? a.V[(q0 + jj) * a.ldv + c] : a.G[(q0 + jj) * a.ldg + c];
        sB[jj][c] = v;
      }
    }
    if (SIDE == 1) {
      for (int jj = tid; jj < BN; jj += kGThreads) {
        const bool in = jj < nb;
        const int64_t t = q0 + jj;
        const float p = in ? (a.row_vec ? a.p_vec[t] : a.p_s) : 0.f;
        sC[jj] = in ? (a.lse[t] - p) * L2E : 0.f;
        sD[jj] = in ? (SMX ? a.delta[t] : a.G[t * a.ldg]) : 0.f;
      }
    }
    __syncthreads();

#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int kb = sb * TM;
      if (kb >= nb) break;
      acc_t s;
#pragma unroll
      for (int r = 0; r < NREG; ++r) s[r] = 0;
#pragma unroll
      for (int st = 0; st < DG; ++st) s = F::mma(sA[kb + q][g * DG + st], pa[st], s);
      acc_t dp;
      if constexpr (SMX) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) dp[r] = 0;
#pragma unroll
        for (int st = 0; st < CG; ++st) dp = F::mma(sB[kb + q][g * CG + st], pb[st], dp);
      }
      float P[NREG], dS[NREG];
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        const int key = kb + F::key_of(r, g);
        bool valid = key < nb;
        if (CONS == C_LOGSUMEXP && a.exclude_self) valid = valid && (q0 + key != o);
        float x = SIDE == 0 ? F::exp2(s[r] - ci) : F::exp2(s[r] * L2E - sC[key]);
        x = valid ? x : 0.f;
        P[r] = x;
        const float dr = SIDE == 0 ? di : sD[key];
        if constexpr (SMX) dS[r] = x * (dp[r] - dr);
        else dS[r] = x * dr;
      }
      // Own-point gradient: sum over the streamed side of dS times its point.
#pragma unroll
      for (int c = 0; c < ND; ++c) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const int ch = c * TM + q;
          const float av = ch < DP ? sA[kb + F::key_of(r, g)][ch] : 0.f;
          oa[c] = F::mma(av, dS[r], oa[c]);
        }
      }
      if constexpr (SMX && SIDE == 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int r = 0; r < NREG; ++r) ob[c] = F::mma(sB[kb + F::key_of(r, g)][c * TM + q], P[r], ob[c]);
        }
      }
    }
  }
  if (!ov) return;
  float *dst = a.partial + ((int64_t)sp * n_own + o) * a.W;
#pragma unroll
  for (int c = 0; c < ND; ++c)
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      const int d = c * TM + F::key_of(r, g);
      if (d < a.D) dst[d] = (SIDE == 0 ? ri : 1.f) * oa[c][r];
    }
  if constexpr (SMX && SIDE == 1) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        const int ch = c * TM + F::key_of(r, g);
        if (ch < a.C) dst[a.D + ch] = ob[c][r];
      }
  }
}

template <int CONS, int DP, int CP>
hipError_t mfma_grad_side(int side, const MfmaGradArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.n_rb * a.n_split)), block(kGThreads);
  if (side == 0) hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 0>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 1>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int CONS, int DP>
hipError_t mfma_grad_cp(int side, int cp, const MfmaGradArgs &a, hipStream_t s) {
  if constexpr (CONS == C_SOFTMAX) {
    if (cp == 32) return mfma_grad_side<CONS, DP, 32>(side, a, s);
    if (cp == 64) return mfma_grad_side<CONS, DP, 64>(side, a, s);
    return hipErrorInvalidValue;
  } else {
    return mfma_grad_side<CONS, DP, 32>(side, a, s);
  }
}

template <int CONS>
hipError_t mfma_grad_dp(int side, int dp, int cp, const MfmaGradArgs &a, hipStream_t s) {
  switch (dp) {
    case 16: return mfma_grad_cp<CONS, 16>(side, cp, a, s);
    case 32: return mfma_grad_cp<CONS, 32>(side, cp, a, s);
    case 64: return mfma_grad_cp<CONS, 64>(side, cp, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int mfma_grad_rows() { return kGWaves * 32; }

hipError_t mfma_grad_launch(int consumer, int side, int dp, int cp, const MfmaGradArgs &a, hipStream_t s) {
  if (consumer == C_SOFTMAX) return mfma_grad_dp<C_SOFTMAX>(side, dp, cp, a, s);
  if (consumer == C_LOGSUMEXP) return mfma_grad_dp<C_LOGSUMEXP>(side, dp, cp, a, s);
  return hipErrorInvalidValue;
}

}  // namespace pw
