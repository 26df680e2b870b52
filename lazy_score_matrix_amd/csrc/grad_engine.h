// Backward tile engine: gradients of sum(consumer output * G) by replaying
// the pairs (torchpairwise guide, opening section and "What to Check",
// Gradients), never storing the [N, M] matrix.
//
// One thread owns one point of one side and streams the other side through
// LDS tiles, like the forward vector engine:
//   SIDE 0  thread = row i, tiles of columns j: dX_i and the row-op grads
//   SIDE 1  thread = column j, tiles of rows i: dY_j, dV_j and the
//           column-op grads
// so every gradient is a private sum (no atomics) over the other side,
// split over column (row) ranges and merged in fixed order.
//
// Per pair: the metric f, the op list replayed left to right keeping every
// intermediate t_k, the consumer's upstream gradient
//   matmul        dS = G_i . V_j                  (dV_j += s G_i)
//   displacement  dS = G_i . (y_j - x_i)          (dX_i -= s G_i, dY_j += s G_i)
//   logsumexp     dS = g_i exp(s - lse_i)
//   softmax@V     dS = P (G_i . V_j - delta_i),  P = exp(s - lse_i)  (dV_j += P G_i)
// then back through the ops (MUL c: d *= c; ADD_ROWS: grad += d;
// WEIGHT_ROWS w: grad += d t_{k-1}, d *= w; EXP: d *= t_k; and the column
// forms) and the metric: with d0 the gradient reaching f,
//   linear       grad(own) += d0 other
//   sqeuclidean  grad(own) += 2 d0 (own - other)
//   rbf          grad(own) += -2 gamma f d0 (own - other)
//   cosine       grad(own) += d0 (-other / (|own||other|) + (own.other) own / (|own|^3 |other|))
// accumulated as sums over `other` and a scalar, finished once per thread.
#pragma once

#include "device_common.h"
#include "pw.h"

namespace pw {

constexpr int kGradBM = 256, kGradBN = 64;

template <class T>
__device__ __forceinline__ T grad_exp(T x) {
  if constexpr (sizeof(T) == 4) return __builtin_amdgcn_exp2f(x * (T)kLog2e);
  else return dexp(x);
}

// FAST: the ops fold into one affine stage s = r_i q_j f + p_i + o_j (the
// forward's canonical stage, vectors precomputed) and no op-vector gradient
// is wanted, so a pair needs no replay of the op list: ds/df = r_i q_j.
template <class T, int METRIC, int CONS, int DT, int CT, int SIDE, bool FAST>
__global__ __launch_bounds__(kGradBM) void grad_tile(const GradArgs a) {
  constexpr int BM = kGradBM, BN = kGradBN, NO = kGradOps;
  constexpr bool HAS_V = CONS == C_MATMUL || CONS == C_SOFTMAX;
  constexpr int GW = HAS_V ? CT : (CONS == C_DISPLACEMENT ? DT : 1);  // G row width
  constexpr int OWNW = SIDE == 0 ? GW : (HAS_V ? CT : 1);             // own value row
  constexpr int OTHW = SIDE == 0 ? (HAS_V ? CT : 1) : GW;             // staged value row
  constexpr bool ROW_LSE = CONS == C_LOGSUMEXP || CONS == C_SOFTMAX;

  __shared__ T sP[BN][DT];     // other points
  __shared__ T sW[BN][OTHW];   // other value rows (V_j on side 0, G_i on side 1)
  __shared__ T sO[NO][BN];     // other side's op vector values
  __shared__ T sL[BN], sDl[BN], sIn[BN];
  __shared__ int sK[BN];       // other side's row / column mask
  __shared__ int64_t sGr[BN];  // other side's group ids
  __shared__ T sA[FAST ? BN : 1], sB[FAST ? BN : 1];  // other side's stage factor and offset

  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb, sp = blockIdx.x / a.n_rb;
  const int64_t n_own = SIDE == 0 ? a.N : a.M, n_oth = SIDE == 0 ? a.M : a.N;
  const int64_t o = (int64_t)rb * BM + tid;
  const bool ov = o < n_own;
  const int64_t qb = (int64_t)sp * a.split, qe = min(n_oth, qb + a.split);
  const T *Own = static_cast<const T *>(SIDE == 0 ? a.X : a.Y);
  const T *Oth = static_cast<const T *>(SIDE == 0 ? a.Y : a.X);
  const int64_t ldown = SIDE == 0 ? a.ldx : a.ldy, ldoth = SIDE == 0 ? a.ldy : a.ldx;
  const T *Gp = static_cast<const T *>(a.G);
  const T *Vp = static_cast<const T *>(a.V);
  const MaskArgs &mk = a.mask;
  const int own_where = SIDE == 0 ? 1 : 2;  // op vectors held per thread

  // ---- own state
  T p[DT], w[OWNW], ownop[NO];
#pragma unroll
  for (int d = 0; d < DT; ++d) p[d] = (ov && d < a.D) ? Own[o * ldown + d] : (T)0;
#pragma unroll
  for (int c = 0; c < OWNW; ++c) {
    T v = 0;
    if (ov) {
      if constexpr (SIDE == 0) {
        if (c < (HAS_V ? a.C : (CONS == C_DISPLACEMENT ? a.D : 1))) v = Gp[o * a.ldg + c];
      } else if constexpr (HAS_V) {
        if (c < a.C) v = Vp[o * a.ldv + c];
      }
    }
    w[c] = v;
  }
#pragma unroll
  for (int t = 0; t < NO; ++t)
    ownop[t] = (ov && t < a.n_ops && a.ops[t].where == own_where) ? static_cast<const T *>(a.ops[t].vec)[o] : (T)0;
  T own_lse = 0, own_dl = 0;
  if constexpr (SIDE == 0 && ROW_LSE) {
    if (ov) {
      own_lse = static_cast<const T *>(a.lse)[o];
      if constexpr (CONS == C_SOFTMAX) own_dl = static_cast<const T *>(a.delta)[o];
    }
  }
  T own_in = 0;
  if constexpr (METRIC == M_COSINE) {
    if (ov) own_in = static_cast<const T *>(SIDE == 0 ? a.inv_x : a.inv_y)[o];
  }
  // FAST stage values of the own side: (r_i, p_i) for rows, (q_j, o_j) for columns.
  T own_a = 1, own_b = 0;
  if constexpr (FAST) {
    const Stage &st = a.stage;
    if (SIDE == 0) {
      if (st.row_vec) {
        if (ov) {
          own_a = static_cast<const T *>(st.r_vec)[o];
          own_b = static_cast<const T *>(st.p_vec)[o];
        }
      } else {
        own_a = (T)st.r_scalar;
        own_b = (T)st.p_scalar;
      }
    } else if (st.col_vec && ov) {
      own_a = static_cast<const T *>(st.q_vec)[o];
      own_b = static_cast<const T *>(st.o_vec)[o];
    }
  }
  const bool own_keep = ov && (SIDE == 0 ? (!mk.row || mk.row[o]) : (!mk.col || mk.col[o]));
  const int64_t own_grp = (ov && mk.grow) ? (SIDE == 0 ? mk.grow[o] : mk.gcol[o]) : 0;
  const T ng = (T)(-a.gamma);

  // ---- accumulators
  T vacc[DT], dacc[DT], vv[HAS_V && SIDE == 1 ? CT : 1], og[NO];
#pragma unroll
  for (int d = 0; d < DT; ++d) vacc[d] = dacc[d] = 0;
#pragma unroll
  for (int c = 0; c < (HAS_V && SIDE == 1 ? CT : 1); ++c) vv[c] = 0;
#pragma unroll
  for (int t = 0; t < NO; ++t) og[t] = 0;
  T sw = 0, ssum = 0;

  for (int64_t q0 = qb; q0 < qe; q0 += BN) {
    const int nb = (int)min((int64_t)BN, qe - q0);
    __syncthreads();
    for (int e = tid; e < BN * DT; e += BM) {
      const int jj = e / DT, d = e % DT;
      sP[jj][d] = (jj < nb && d < a.D) ? Oth[(q0 + jj) * ldoth + d] : (T)0;
    }
    for (int e = tid; e < BN * OTHW; e += BM) {
      const int jj = e / OTHW, c = e % OTHW;
      T v = 0;
      if (jj < nb) {
        if constexpr (SIDE == 1) {
          if (c < (HAS_V ? a.C : (CONS == C_DISPLACEMENT ? a.D : 1))) v = Gp[(q0 + jj) * a.ldg + c];
        } else if constexpr (HAS_V) {
          if (c < a.C) v = Vp[(q0 + jj) * a.ldv + c];
        }
      }
      sW[jj][c] = v;
    }
    for (int e = tid; e < NO * BN; e += BM) {
      const int t = e / BN, jj = e % BN;
      if (t < a.n_ops && a.ops[t].where == 3 - own_where)
        sO[t][jj] = jj < nb ? static_cast<const T *>(a.ops[t].vec)[q0 + jj] : (T)0;
    }
    for (int jj = tid; jj < BN; jj += BM) {
      const bool in = jj < nb;
      const int64_t q = q0 + jj;
      if constexpr (SIDE == 1 && ROW_LSE) {
        sL[jj] = in ? static_cast<const T *>(a.lse)[q] : (T)0;
        sDl[jj] = (in && CONS == C_SOFTMAX) ? static_cast<const T *>(a.delta)[q] : (T)0;
      }
      if constexpr (METRIC == M_COSINE) sIn[jj] = in ? static_cast<const T *>(SIDE == 0 ? a.inv_y : a.inv_x)[q] : (T)0;
      sK[jj] = in && (SIDE == 0 ? (!mk.col || mk.col[q]) : (!mk.row || mk.row[q]));
      if constexpr (FAST) {
        const Stage &st = a.stage;
        T va = 1, vb = 0;
        if (SIDE == 0) {
          if (st.col_vec && in) {
            va = static_cast<const T *>(st.q_vec)[q];
            vb = static_cast<const T *>(st.o_vec)[q];
          }
        } else if (st.row_vec) {
          if (in) {
            va = static_cast<const T *>(st.r_vec)[q];
            vb = static_cast<const T *>(st.p_vec)[q];
          }
        } else {
          va = (T)st.r_scalar;
          vb = (T)st.p_scalar;
        }
        sA[jj] = va;
        sB[jj] = vb;
      }
      sGr[jj] = (in && mk.grow) ? (SIDE == 0 ? mk.gcol[q] : mk.grow[q]) : 0;
    }
    __syncthreads();
    if (!own_keep) continue;

    for (int jj = 0; jj < nb; ++jj) {
      const int64_t q = q0 + jj;
      const int64_t i = SIDE == 0 ? o : q, j = SIDE == 0 ? q : o;
      if (!sK[jj]) continue;
      if (mk.any && !pair_kept(mk, i, j, SIDE == 0 ? own_grp : sGr[jj], SIDE == 0 ? sGr[jj] : own_grp)) continue;
      if (CONS == C_LOGSUMEXP && a.exclude_self && i == j) continue;

      // metric
      T f, dot = 0;
      {
        T acc = 0;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          if constexpr (METRIC == M_LINEAR || METRIC == M_COSINE) {
            acc = fma(p[d], sP[jj][d], acc);
          } else {
            const T df = p[d] - sP[jj][d];
            acc = fma(df, df, acc);
          }
        }
        if constexpr (METRIC == M_LINEAR) f = acc;
        else if constexpr (METRIC == M_SQEUCLIDEAN) f = acc;
        else if constexpr (METRIC == M_RBF) f = grad_exp(ng * acc);
        else {
          dot = acc;
          f = fma(-dot * own_in, sIn[jj], (T)1);
        }
      }
      // forward through the ops, keeping every intermediate
      T tv[NO + 1];
      tv[0] = f;
      T Rq = 1;
      if constexpr (FAST) {
        Rq = own_a * sA[jj];
        tv[NO] = fma(f, Rq, own_b + sB[jj]);
      }
#pragma unroll
      for (int t = 0; t < NO; ++t) {
        if constexpr (FAST) break;
        T x = tv[t];
        if (t < a.n_ops) {
          const int kind = a.ops[t].kind;
          const T vec_v = a.ops[t].where == own_where ? ownop[t] : sO[t][jj];
          if (kind == PW_OP_MUL) x = (T)a.ops[t].scalar * x;
          else if (kind == PW_OP_ADD) x = x + (T)a.ops[t].scalar;
          else if (kind == PW_OP_ADD_ROWS || kind == PW_OP_ADD_COLUMNS) x = x + vec_v;
          else if (kind == PW_OP_WEIGHT_ROWS || kind == PW_OP_WEIGHT_COLUMNS) x = vec_v * x;
          else if (kind == PW_OP_EXP) x = grad_exp(x);
        }
        tv[t + 1] = x;
      }
      const T s = tv[NO];

      // upstream gradient of the pair and the direct terms
      T dS;
      if constexpr (CONS == C_MATMUL) {
        T acc = 0;
#pragma unroll
        for (int c = 0; c < CT; ++c) acc = fma(w[c], sW[jj][c], acc);
        dS = acc;
        if constexpr (SIDE == 1) {
#pragma unroll
          for (int c = 0; c < CT; ++c) vv[c] = fma(s, sW[jj][c], vv[c]);
        }
      } else if constexpr (CONS == C_DISPLACEMENT) {
        T acc = 0;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const T gi = SIDE == 0 ? w[d] : sW[jj][d];
          const T xi = SIDE == 0 ? p[d] : sP[jj][d];
          const T yj = SIDE == 0 ? sP[jj][d] : p[d];
          acc = fma(gi, yj - xi, acc);
          if constexpr (SIDE == 1) dacc[d] = fma(s, gi, dacc[d]);
        }
        dS = acc;
        if constexpr (SIDE == 0) ssum += s;
      } else if constexpr (CONS == C_LOGSUMEXP) {
        const T gi = SIDE == 0 ? w[0] : sW[jj][0];
        const T li = SIDE == 0 ? own_lse : sL[jj];
        dS = gi * grad_exp(s - li);
      } else {
        const T li = SIDE == 0 ? own_lse : sL[jj];
        const T di = SIDE == 0 ? own_dl : sDl[jj];
        const T P = grad_exp(s - li);
        T acc = 0;
#pragma unroll
        for (int c = 0; c < CT; ++c) acc = fma(w[c], sW[jj][c], acc);
        dS = P * (acc - di);
        if constexpr (SIDE == 1) {
#pragma unroll
          for (int c = 0; c < CT; ++c) vv[c] = fma(P, sW[jj][c], vv[c]);
        }
      }

      // back through the ops
      T dd = dS;
      if constexpr (FAST) dd = dS * Rq;
#pragma unroll
      for (int t = NO - 1; t >= 0; --t) {
        if constexpr (FAST) break;
        if (t < a.n_ops) {
          const int kind = a.ops[t].kind;
          const bool mine = a.ops[t].where == own_where;
          const T vec_v = mine ? ownop[t] : sO[t][jj];
          if (kind == PW_OP_MUL) {
            dd = (T)a.ops[t].scalar * dd;
          } else if (kind == PW_OP_ADD_ROWS || kind == PW_OP_ADD_COLUMNS) {
            if (mine) og[t] += dd;
          } else if (kind == PW_OP_WEIGHT_ROWS || kind == PW_OP_WEIGHT_COLUMNS) {
            if (mine) og[t] = fma(dd, tv[t], og[t]);
            dd = vec_v * dd;
          } else if (kind == PW_OP_EXP) {
            dd = dd * tv[t + 1];
          }
        }
      }

      // metric gradient sums
      T c1, c2;
      if constexpr (METRIC == M_LINEAR) {
        c1 = dd;
        c2 = 0;
      } else if constexpr (METRIC == M_SQEUCLIDEAN) {
        c1 = (T)2 * dd;
        c2 = c1;
      } else if constexpr (METRIC == M_RBF) {
        c1 = (T)(-2 * a.gamma) * f * dd;
        c2 = c1;
      } else {
        c1 = dd * sIn[jj];
        c2 = c1 * dot;
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) vacc[d] = fma(c1, sP[jj][d], vacc[d]);
      sw += c2;
    }
  }
  if (!ov) return;

  // finish: gradient of the own point
  T gown[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) {
    T g;
    if constexpr (METRIC == M_LINEAR) g = vacc[d];
    else if constexpr (METRIC == M_COSINE) g = fma(sw * own_in * own_in * own_in, p[d], -own_in * vacc[d]);
    else g = fma(sw, p[d], -vacc[d]);
    if constexpr (CONS == C_DISPLACEMENT) g = SIDE == 0 ? fma(-ssum, w[d], g) : g + dacc[d];
    gown[d] = g;
  }
  T *out = static_cast<T *>(a.partial) + ((int64_t)sp * n_own + o) * a.W;
#pragma unroll
  for (int d = 0; d < DT; ++d)
    if (d < a.D) out[d] = gown[d];
  int at = a.D;
  if constexpr (HAS_V && SIDE == 1) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
      if (c < a.C) out[at + c] = vv[c];
    at += a.C;
  }
#pragma unroll
  for (int t = 0; t < NO; ++t)
    if (t < a.n_ops) out[at + t] = og[t];
}

// Top-k: gradients flow through the selected pairs only. One thread per row
// replays its k pairs: dX_i and the row-op grads directly, dY_j and the
// column-op grads with atomic adds into outputs cleared beforehand.
template <class T, int METRIC, int DT>
__global__ __launch_bounds__(kGradBM) void grad_topk(const GradArgs a) {
  constexpr int NO = kGradOps;
  const int64_t i = (int64_t)blockIdx.x * kGradBM + threadIdx.x;
  if (i >= a.N) return;
  const T *X = static_cast<const T *>(a.X);
  const T *Y = static_cast<const T *>(a.Y);
  const T *Gp = static_cast<const T *>(a.G);
  T x[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) x[d] = d < a.D ? X[i * a.ldx + d] : (T)0;
  const T inx = METRIC == M_COSINE ? static_cast<const T *>(a.inv_x)[i] : (T)0;
  T gx[DT], og[NO];
  T vacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) gx[d] = vacc[d] = 0;
#pragma unroll
  for (int t = 0; t < NO; ++t) og[t] = 0;
  T sw = 0;
  for (int pk = 0; pk < a.k; ++pk) {
    const int64_t j = a.idx[i * a.k + pk];
    if (j < 0 || j >= a.M) continue;  // empty slot (or not an index of this score)
    T y[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d) y[d] = d < a.D ? Y[j * a.ldy + d] : (T)0;
    T acc = 0;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      if constexpr (METRIC == M_LINEAR || METRIC == M_COSINE) acc = fma(x[d], y[d], acc);
      else acc = fma(x[d] - y[d], x[d] - y[d], acc);
    }
    const T iny = METRIC == M_COSINE ? static_cast<const T *>(a.inv_y)[j] : (T)0;
    T f;
    if constexpr (METRIC == M_RBF) f = grad_exp((T)(-a.gamma) * acc);
    else if constexpr (METRIC == M_COSINE) f = fma(-acc * inx, iny, (T)1);
    else f = acc;
    T tv[NO + 1];
    tv[0] = f;
#pragma unroll
    for (int t = 0; t < NO; ++t) {
      T v = tv[t];
      if (t < a.n_ops) {
        const GradOp &op = a.ops[t];
        const T vec_v = op.where == 1 ? static_cast<const T *>(op.vec)[i]
                                      : (op.where == 2 ? static_cast<const T *>(op.vec)[j] : (T)0);
        if (op.kind == PW_OP_MUL) v = (T)op.scalar * v;
        else if (op.kind == PW_OP_ADD) v = v + (T)op.scalar;
        else if (op.kind == PW_OP_ADD_ROWS || op.kind == PW_OP_ADD_COLUMNS) v = v + vec_v;
        else if (op.kind == PW_OP_WEIGHT_ROWS || op.kind == PW_OP_WEIGHT_COLUMNS) v = vec_v * v;
        else if (op.kind == PW_OP_EXP) v = grad_exp(v);
      }
      tv[t + 1] = v;
    }
    T dd = Gp[i * a.ldg + pk];
#pragma unroll
    for (int t = NO - 1; t >= 0; --t) {
      if (t < a.n_ops) {
        const GradOp &op = a.ops[t];
        const T vec_v = op.where == 1 ? static_cast<const T *>(op.vec)[i]
                                      : (op.where == 2 ? static_cast<const T *>(op.vec)[j] : (T)0);
        if (op.kind == PW_OP_MUL) {
          dd = (T)op.scalar * dd;
        } else if (op.kind == PW_OP_ADD_ROWS) {
          og[t] += dd;
        } else if (op.kind == PW_OP_ADD_COLUMNS) {
          if (a.dop[t]) atomicAdd(static_cast<T *>(a.dop[t]) + j, dd);
        } else if (op.kind == PW_OP_WEIGHT_ROWS) {
          og[t] = fma(dd, tv[t], og[t]);
          dd = vec_v * dd;
        } else if (op.kind == PW_OP_WEIGHT_COLUMNS) {
          if (a.dop[t]) atomicAdd(static_cast<T *>(a.dop[t]) + j, dd * tv[t]);
          dd = vec_v * dd;
        } else if (op.kind == PW_OP_EXP) {
          dd = dd * tv[t + 1];
        }
      }
    }
    // metric: row side summed here, column side added atomically
    T c1, c2;
    if constexpr (METRIC == M_LINEAR) { c1 = dd; c2 = 0; }
    else if constexpr (METRIC == M_SQEUCLIDEAN) { c1 = (T)2 * dd; c2 = c1; }
    else if constexpr (METRIC == M_RBF) { c1 = (T)(-2 * a.gamma) * f * dd; c2 = c1; }
    else { c1 = dd * iny; c2 = c1 * acc; }
#pragma unroll
    for (int d = 0; d < DT; ++d) vacc[d] = fma(c1, y[d], vacc[d]);
    sw += c2;
    if (a.dY) {
      T *dy = static_cast<T *>(a.dY) + j * a.lddy;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        if (d >= a.D) continue;
        T g;
        if constexpr (METRIC == M_LINEAR) g = dd * x[d];
        else if constexpr (METRIC == M_COSINE) g = dd * (-inx * iny * x[d] + acc * inx * iny * iny * iny * y[d]);
        else g = c1 * (y[d] - x[d]);
        atomicAdd(dy + d, g);
      }
    }
  }
  if (a.dX) {
    T *dx = static_cast<T *>(a.dX) + i * a.lddx;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      if (d >= a.D) continue;
      T g;
      if constexpr (METRIC == M_LINEAR) g = vacc[d];
      else if constexpr (METRIC == M_COSINE) g = fma(sw * inx * inx * inx, x[d], -inx * vacc[d]);
      else g = fma(sw, x[d], -vacc[d]);
      dx[d] = g;
    }
  }
#pragma unroll
  for (int t = 0; t < NO; ++t)
    if (t < a.n_ops && a.ops[t].where == 1 && a.dop[t]) static_cast<T *>(a.dop[t])[i] = og[t];
}

template <class T, int METRIC, int CONS, int DT, int CT>
hipError_t grad_launch_side(int side, const GradArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.n_rb * a.n_split)), block(kGradBM);
  if (a.fast) {
    if (side == 0) hipLaunchKernelGGL((grad_tile<T, METRIC, CONS, DT, CT, 0, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((grad_tile<T, METRIC, CONS, DT, CT, 1, true>), grid, block, 0, s, a);
  } else {
    if (side == 0) hipLaunchKernelGGL((grad_tile<T, METRIC, CONS, DT, CT, 0, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((grad_tile<T, METRIC, CONS, DT, CT, 1, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <class T, int METRIC, int DT>
hipError_t grad_by_consumer(int consumer, int side, int ct, const GradArgs &a, hipStream_t s) {
  switch (consumer) {
    case C_MATMUL:
      return ct == 16 ? grad_launch_side<T, METRIC, C_MATMUL, DT, 16>(side, a, s)
                      : grad_launch_side<T, METRIC, C_MATMUL, DT, 64>(side, a, s);
    case C_SOFTMAX:
      return ct == 16 ? grad_launch_side<T, METRIC, C_SOFTMAX, DT, 16>(side, a, s)
                      : grad_launch_side<T, METRIC, C_SOFTMAX, DT, 64>(side, a, s);
    case C_DISPLACEMENT: return grad_launch_side<T, METRIC, C_DISPLACEMENT, DT, 1>(side, a, s);
    case C_LOGSUMEXP: return grad_launch_side<T, METRIC, C_LOGSUMEXP, DT, 1>(side, a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC>
hipError_t grad_launch_metric(int consumer, int side, int dt, int ct, const GradArgs &a, hipStream_t s) {
  switch (dt) {
    case 4: return grad_by_consumer<T, METRIC, 4>(consumer, side, ct, a, s);
    case 16: return grad_by_consumer<T, METRIC, 16>(consumer, side, ct, a, s);
    case 64: return grad_by_consumer<T, METRIC, 64>(consumer, side, ct, a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC>
hipError_t grad_topk_metric(int dt, const GradArgs &a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + kGradBM - 1) / kGradBM)), block(kGradBM);
  switch (dt) {
    case 4: hipLaunchKernelGGL((grad_topk<T, METRIC, 4>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((grad_topk<T, METRIC, 16>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((grad_topk<T, METRIC, 64>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pw
