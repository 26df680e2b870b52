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
// partial sums that the shared merge kernel adds in split order. A band
// limits the streamed range and classifies tiles like the forward (skipped,
// kept whole, or checked pair by pair, as are row and column masks).
#include "mfma_engine.h"

namespace pw {
namespace {

constexpr int kGWaves = 4, kGThreads = 256, kGBN = 64;

template <int CONS, int DP, int CP, int SIDE, bool MASKED>
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
  __shared__ int sK[MASKED ? BN : 1];                               // streamed side's row / column mask

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, q = l & 31;
  constexpr int OWN = kGWaves * TM;  // own rows (columns) per block
  const int64_t n_own = SIDE == 0 ? a.N : a.M, n_oth = SIDE == 0 ? a.M : a.N;
  const MaskArgs &mk = a.mask;
  // The streamed range a band leaves to own block b: keys j in [i + lo,
  // i + hi] of its rows (row side), rows i in [j - hi, j - lo] of its
  // columns (column side); the start on a tile boundary.
  auto reach = [&](int b, int64_t *f, int64_t *e) {
    const int64_t b0 = (int64_t)b * OWN, b1 = min(n_own, b0 + OWN) - 1;
    int64_t lo = 0, hi = n_oth;
    if (MASKED && mk.band) {
      lo = max(lo, SIDE == 0 ? b0 + mk.lo : b0 - mk.hi);
      hi = min(hi, SIDE == 0 ? b1 + mk.hi + 1 : b1 - mk.lo + 1);
    }
    *f = lo / BN * BN;
    *e = hi;
  };
  // Paired launches (a band): a workgroup takes own blocks r and
  // n_rb - 1 - r and an equal run of their tiles, as the forward does.
  const bool paired = MASKED && a.rb_pairs;
  const int slots = paired ? a.rb_pairs : a.n_rb;
  // XCD-major numbering (workgroups are dealt round-robin to the 8 XCDs) and
  // block coordinates in scalar registers, as in the forward engine.
  const int nblk = gridDim.x;
  const int bid = (nblk % 8 == 0) ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
  const int rb_first = __builtin_amdgcn_readfirstlane(bid % slots);
  const int sp = __builtin_amdgcn_readfirstlane(bid / slots);
  const int npass = MASKED ? ((paired && a.n_rb - 1 - rb_first != rb_first) ? 2 : 1) : 1;
  int64_t pf[2] = {0, 0}, pe[2] = {0, 0}, pt[2] = {0, 0}, v0 = 0, v1 = 0;
  if (paired) {
    for (int p = 0; p < npass; ++p) {
      reach(p ? a.n_rb - 1 - rb_first : rb_first, &pf[p], &pe[p]);
      pt[p] = pe[p] > pf[p] ? (pe[p] - pf[p] + BN - 1) / BN : 0;
    }
    v0 = (pt[0] + pt[1]) * sp / a.n_split;
    v1 = (pt[0] + pt[1]) * (sp + 1) / a.n_split;
  }
  for (int pass = 0; pass < npass; ++pass) {
  const int rb = pass ? a.n_rb - 1 - rb_first : rb_first;
  const int64_t own0 = (int64_t)rb * OWN, own1 = min(n_own, own0 + OWN) - 1;
  const int64_t o = own0 + w * TM + q;
  const bool ov = o < n_own;
  int64_t qb, qe;
  if (paired) {
    const int64_t off = pass ? pt[0] : 0;
    const int64_t t0 = max(v0 - off, (int64_t)0), t1 = min(v1 - off, pt[pass]);
    qb = pf[pass] + t0 * BN;
    qe = t1 > t0 ? min(pe[pass], pf[pass] + t1 * BN) : qb;
  } else {
    qb = (int64_t)sp * a.split;
    qe = min(n_oth, qb + a.split);
    if constexpr (MASKED) {
      int64_t f, e;
      reach(rb, &f, &e);
      if (f > qb) qb += (f - qb) / BN * BN;
      qe = min(qe, e);
    }
  }
  // Own row (column) dropped by the row (column) mask: no pair contributes.
  const bool own_keep = ov && (!MASKED || (SIDE == 0 ? (!mk.row || mk.row[o]) : (!mk.col || mk.col[o])));

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

  qb = wave_uniform(qb);
  qe = wave_uniform(qe);
  // Row side: streamed tiles come through registers, the global reads of the
  // next tile (16-byte vectors from a uniform base when the tile is full and
  // aligned) in flight while the current tile is computed from LDS. The
  // column side holds twice the accumulators and has no registers to spare
  // for that: it reads each tile between the tile's two barriers, four
  // features at a time.
  constexpr bool PF = SIDE == 0;
  TileLoader<float, BN, DP, kGThreads> ldA;
  TileLoader<float, BN, CPS, kGThreads> ldB;
  if constexpr (PF) {
    ldA.init(a.ldy, vec_ok(a.Y, a.ldy, 4), tid);
    if constexpr (SMX) ldB.init(a.ldv, vec_ok(a.V, a.ldv, 4), tid);
  }
  auto fetch = [&](int64_t t0) {
    if constexpr (PF) {
      const int nbt = (int)min((int64_t)BN, qe - t0);
      ldA.load(a.Y, a.ldy, t0, nbt, a.D, tid);
      if constexpr (SMX) ldB.load(a.V, a.ldv, t0, nbt, a.C, tid);
    }
  };
  if (qb < qe) fetch(qb);
  for (int64_t q0 = qb; q0 < qe; q0 += BN) {
    const int nb = (int)min((int64_t)BN, qe - q0);
    const bool next = q0 + BN < qe;
    // Tile class under the masks (uniform over the workgroup): skipped
    // tiles are not staged; boundary tiles check every pair.
    bool check = false;
    if (MASKED) {
      const int64_t s1 = q0 + nb - 1;
      const int cls = SIDE == 0 ? tile_class(mk, own0, own1, q0, s1, 0, 0) : tile_class(mk, q0, s1, own0, own1, 0, 0);
      if (cls == TILE_SKIP) {
        if (next) fetch(q0 + BN);
        continue;
      }
      check = cls != TILE_FULL || mk.row || mk.col;
    }
    __syncthreads();  // every wave is done with the previous tile
    if constexpr (PF) {
      ldA.store(sA, tid);
      if constexpr (SMX) ldB.store(sB, tid);
    } else {
      // Four consecutive features per thread and step: one 16-byte read
      // when the rows are aligned and unpadded, else element by element.
      typedef float f4 __attribute__((ext_vector_type(4)));
      const bool xv = vec_ok(a.X, a.ldx, 4) && a.D == DP;
#pragma unroll
      for (int e = tid; e < BN * DP / 4; e += kGThreads) {
        const int jj = e / (DP / 4), d = (e % (DP / 4)) * 4;
        f4 v = {0.f, 0.f, 0.f, 0.f};
        if (jj < nb) {
          const int64_t t = q0 + jj;
          const float *src = a.X + t * a.ldx + d;
          if (xv) {
            v = *reinterpret_cast<const f4 *>(src);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = d + u < a.D ? src[u] : 0.f;
          }
          v *= a.row_vec ? a.r_vec[t] : a.r_s;
        }
        *reinterpret_cast<f4 *>(&sA[jj][d]) = v;
      }
      if constexpr (SMX) {
        const bool gv = vec_ok(a.G, a.ldg, 4) && a.C == CP;
#pragma unroll
        for (int e = tid; e < BN * CP / 4; e += kGThreads) {
          const int jj = e / (CP / 4), c = (e % (CP / 4)) * 4;
          f4 v = {0.f, 0.f, 0.f, 0.f};
          if (jj < nb) {
            const float *src = a.G + (q0 + jj) * a.ldg + c;
            if (gv) {
              v = *reinterpret_cast<const f4 *>(src);
            } else {
#pragma unroll
              for (int u = 0; u < 4; ++u) v[u] = c + u < a.C ? src[u] : 0.f;
            }
          }
          *reinterpret_cast<f4 *>(&sB[jj][c]) = v;
        }
      }
      for (int jj = tid; jj < BN; jj += kGThreads) {
        const bool in = jj < nb;
        const int64_t t = q0 + jj;
        const float p = in ? (a.row_vec ? a.p_vec[t] : a.p_s) : 0.f;
        sC[jj] = in ? (a.lse[t] - p) * L2E : 0.f;
        sD[jj] = in ? (SMX ? a.delta[t] : a.G[t * a.ldg]) : 0.f;
      }
    }
    if (MASKED && check) {  // the streamed side's row / column mask
      for (int jj = tid; jj < BN; jj += kGThreads) {
        const int64_t t = q0 + jj;
        sK[MASKED ? jj : 0] = jj < nb && (SIDE == 0 ? (!mk.col || mk.col[t]) : (!mk.row || mk.row[t]));
      }
    }
    if (next) fetch(q0 + BN);
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
        P[r] = SIDE == 0 ? F::exp2(s[r] - ci) : F::exp2(s[r] * L2E - sC[key]);
      }
      // Pairs are dropped only in ragged sub-blocks, sub-blocks that may
      // hold the own point itself (exclude_self) and checked tiles: a branch
      // marked unlikely keeps that test off every other sub-block (left to
      // itself the compiler turns it into a select on every register). An
      // own row (column) dropped by its mask is zeroed at the store instead:
      // a lane's dS only ever reaches its own outputs.
      const bool ragged = kb + TM > nb;
      const bool self = CONS == C_LOGSUMEXP && a.exclude_self && q0 + kb <= own1 && q0 + kb + TM > own0;
      if (__builtin_expect(ragged || self || (MASKED && check), 0)) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const int key = kb + F::key_of(r, g);
          bool valid = key < nb;
          if (CONS == C_LOGSUMEXP && a.exclude_self) valid = valid && (q0 + key != o);
          if (MASKED && check) {
            const int64_t i = SIDE == 0 ? o : q0 + key, j = SIDE == 0 ? q0 + key : o;
            valid = valid && sK[MASKED ? key : 0] && pair_kept(mk, i, j, 0, 0);
          }
          P[r] = valid ? P[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        const int key = kb + F::key_of(r, g);
        const float dr = SIDE == 0 ? di : sD[key];
        if constexpr (SMX) dS[r] = P[r] * (dp[r] - dr);
        else dS[r] = P[r] * dr;
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
  if (!MASKED && !ov) return;  // one pass only: nothing follows
  if (ov) {
    float *dst = a.partial + ((int64_t)sp * n_own + o) * a.W;
#pragma unroll
    for (int c = 0; c < ND; ++c)
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        const int d = c * TM + F::key_of(r, g);
        if (d < a.D) dst[d] = own_keep ? (SIDE == 0 ? ri : 1.f) * oa[c][r] : 0.f;
      }
    if constexpr (SMX && SIDE == 1) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const int ch = c * TM + F::key_of(r, g);
          if (ch < a.C) dst[a.D + ch] = own_keep ? ob[c][r] : 0.f;
        }
    }
  }
  }  // pass
}

template <int CONS, int DP, int CP>
hipError_t mfma_grad_side(int side, const MfmaGradArgs &a, hipStream_t s) {
  const int slots = (a.mask.any && a.rb_pairs) ? a.rb_pairs : a.n_rb;
  dim3 grid((unsigned)(slots * a.n_split)), block(kGThreads);
  if (a.mask.any) {
    if (side == 0) hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 0, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 1, true>), grid, block, 0, s, a);
  } else {
    if (side == 0) hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 0, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((mfma_grad_kernel<CONS, DP, CP, 1, false>), grid, block, 0, s, a);
  }
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
