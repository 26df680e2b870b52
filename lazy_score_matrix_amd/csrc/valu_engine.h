// Generic VALU tile engine.
//
// One thread owns one row x_i (kept in registers) and streams the columns of
// its workgroup's column range through LDS tiles of kValuBN rows of Y (and V
// and the staged column epilogue vectors). Every lane of a wave reads the
// same LDS address for a column, so the reads are broadcasts. Each score is
// evaluated in direct form (the sum of squared differences for the distance
// metrics, so identical points are at distance exactly 0 however far from
// the origin; the dot product scaled by 1/|x_i| and a staged 1/|y_j| for
// cosine), run through the epilogue, and folded into the row's reduction:
//   matmul        acc[c] += s * V[j, c]
//   displacement  acc[d] += s * y_jd, mass += s; out = acc - x * mass
//   logsumexp     online (max m, sum l) per group of 8 columns
//   softmax@V     online (m, l, acc[c]) per group of 8 columns
//   top-k         sorted register list of (value, index) keys behind a
//                 value threshold; k = 1 keeps one (value, index) pair
// This engine covers every D in 1..64, every op chain and both dtypes; the
// planner prefers it for small D and small value widths, where there is no
// real contraction to hand to the matrix cores.
#pragma once

#include "device_common.h"

namespace pw {

// neg_gamma = -gamma for double (device exp); -gamma * log2(e) for float
// (the hardware base-2 exponential). PRE: float rbf with both points
// pre-scaled by sqrt(gamma log2(e)), so the squared distance is the
// exponent itself (identical points still give exactly 1).
template <int METRIC, class T, int DT, bool PRE = false>
__device__ __forceinline__ T valu_metric(const T (&x)[DT], const T *y, T neg_gamma) {
  if constexpr (METRIC == M_LINEAR || METRIC == M_COSINE) {
    if constexpr (DT <= 4) {
      T s = x[0] * y[0];
#pragma unroll
      for (int d = 1; d < DT; ++d) s = fma(x[d], y[d], s);
      return s;
    }
    T s0 = 0, s1 = 0;
#pragma unroll
    for (int d = 0; d < DT; d += 2) {
      s0 = fma(x[d], y[d], s0);
      if (d + 1 < DT) s1 = fma(x[d + 1], y[d + 1], s1);
    }
    return s0 + s1;
  } else {
    T d2;
    if constexpr (DT <= 4) {
      // One chain: the columns of a tile already give the ILP.
      T t = x[0] - y[0];
      d2 = t * t;
#pragma unroll
      for (int d = 1; d < DT; ++d) {
        t = x[d] - y[d];
        d2 = fma(t, t, d2);
      }
    } else {
      T s0 = 0, s1 = 0;
#pragma unroll
      for (int d = 0; d < DT; d += 2) {
        T t0 = x[d] - y[d];
        s0 = fma(t0, t0, s0);
        if (d + 1 < DT) {
          T t1 = x[d + 1] - y[d + 1];
          s1 = fma(t1, t1, s1);
        }
      }
      d2 = s0 + s1;
    }
    if constexpr (METRIC == M_RBF) {
      if constexpr (PRE) return __builtin_amdgcn_exp2f(-d2);
      if constexpr (sizeof(T) == 4) return __builtin_amdgcn_exp2f(neg_gamma * d2);
      else return dexp(neg_gamma * d2);
    }
    return d2;
  }
}

template <class T, int METRIC, int CONS, int DT, int VT>
__global__ __launch_bounds__(kValuBM) void valu_tile(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  constexpr int BM = kValuBM, BN = kValuBN;
  constexpr bool HAS_V = (CONS == C_MATMUL || CONS == C_SOFTMAX);
  constexpr int VW = HAS_V ? VT : 1;
  constexpr int ACCN = HAS_V ? VT : (CONS == C_DISPLACEMENT ? DT : 1);
  constexpr int KL = (CONS == C_TOPK) ? VT : 1;
  constexpr int G = 8;  // columns per online-softmax or top-k screening group
  // Three features are stored unpadded: four consecutive columns are three
  // 16-byte reads, and every broadcast read costs the LDS its full width.
  constexpr int DTS = DT;

  __shared__ T sY[BN][DTS];
  __shared__ T sV[BN][VW];
  __shared__ T sQ[kMaxStages][BN];
  __shared__ T sO[kMaxStages][BN];
  __shared__ T sR[METRIC == M_COSINE ? BN : 1];  // 1/|y_j| for cosine
  __shared__ int sC[BN];                          // column mask flags
  __shared__ int64_t sG[BN];                      // column group ids

  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb;
  const int sp = blockIdx.x / a.n_rb;
  const int64_t i = (int64_t)rb * BM + tid;
  const bool rv = i < a.N;
  const int64_t jb = (int64_t)sp * a.split_cols;
  const int64_t je = min(a.M, jb + a.split_cols);
  const MaskArgs &mk = a.mask;
  const int64_t r0 = (int64_t)rb * BM, r1 = min(a.N, r0 + BM) - 1;
  const bool rkeep = rv && (!mk.row || mk.row[i]);
  const int64_t gi = (rv && mk.grow) ? mk.grow[i] : 0;
  int64_t jfirst, jlast;
  band_range(mk, rb, r0, r1, jb, je, BN, &jfirst, &jlast);
  // The column range is the workgroup's: keep it (and so every column
  // index) in scalar registers.
  jfirst = wave_uniform(jfirst);
  jlast = wave_uniform(jlast);

  // Float rbf (but displacement, which needs the coordinates themselves)
  // scales both sides by sqrt(gamma log2(e)) once, which saves the
  // multiply of every pair's exponent.
  constexpr bool PRE = METRIC == M_RBF && sizeof(T) == 4 && CONS != C_DISPLACEMENT;
  const T pre_s = PRE ? (T)sqrt(a.gamma * kLog2e) : (T)1;
  T x[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) x[d] = (rv && d < a.D) ? ldg<T>(bp.X, i * a.ldx + d) * pre_s : (T)0;
  RowEpi<T> re;
  load_row_epi<T>(a.epi, i, rv, re, epi_shift(a));
  const T neg_gamma = sizeof(T) == 4 ? (T)(-a.gamma * kLog2e) : (T)(-a.gamma);
  T rx = 0;  // 1/|x_i| for cosine (0 for a zero row)
  if constexpr (METRIC == M_COSINE) {
    T n2 = 0;
#pragma unroll
    for (int d = 0; d < DT; ++d) n2 = fma(x[d], x[d], n2);
    rx = n2 > (T)0 ? (T)1 / sqrt(n2) : (T)0;
  }
  // Whether column slot jj of the tile at j0 (a checked tile) survives the
  // masks.
  int64_t j0c = 0;
  auto kept = [&](int jj) -> bool { return sC[jj] && pair_kept(a.mask, i, j0c + jj, gi, sG[jj]); };
  // Score of column slot jj (the metric; cosine scales the dot product).
  auto metric = [&](int jj) -> T {
    T v = valu_metric<METRIC, T, DT, PRE>(x, sY[jj], neg_gamma);
    if constexpr (METRIC == M_COSINE) v = fma(-v * sR[jj], rx, (T)1);
    return v;
  };

  T acc[ACCN];
#pragma unroll
  for (int c = 0; c < ACCN; ++c) acc[c] = 0;
  T mass = 0;
  T m = neg_inf<T>(), l = 0;
  // Online consumers in float with at most one row-only affine stage run in
  // base 2 (m is then a base-2 maximum until the end of the sweep).
  const bool fast2 = (CONS == C_LOGSUMEXP || CONS == C_SOFTMAX) && sizeof(T) == 4 &&
                     (a.epi.n_stages == 0 ||
                      (a.epi.n_stages == 1 && a.epi.st[0].kind == ST_AFFINE && !a.epi.st[0].col_vec));
  const T r2 = (T)kLog2e * (a.epi.n_stages ? re.r[0] : (T)1);
  const T p2 = (T)kLog2e * (a.epi.n_stages ? re.p[0] : (T)0);
  T q2 = p2;  // p2 less the base-2 reference (0 until there is one)
  // Top-k list in the signed orientation (negated for `largest`): values
  // ascending, equal values in column order, empty slots at +inf with column
  // ~0; thr is the last value. With k = 1 the best signed value and its
  // column are kept directly (thr, best_j).
  T lv[KL];
  uint32_t lj[KL];
#pragma unroll
  for (int p = 0; p < KL; ++p) {
    lv[p] = (T)__builtin_huge_val();
    lj[p] = ~0u;
  }
  T thr = __builtin_huge_val();
  uint32_t best_j = ~0u;
  // k > 1: candidates below the threshold (as it stood when they were met)
  // are queued in LDS, one column of slots per lane, and the whole wave
  // inserts them together once some lane's queue could overflow, and at the
  // end. An insertion then runs once per queued candidate of the wave's
  // fullest lane, instead of once for every column at which any lane had a
  // candidate. A candidate enters only if still below the threshold when
  // its turn comes; queues keep column order, so ties still go to the
  // lower index.
  constexpr bool QUEUE = CONS == C_TOPK && KL > 1;
  constexpr int QCAP = QUEUE ? (sizeof(T) == 4 ? 16 : 12) : 1;
  static_assert(!QUEUE || QCAP >= G, "a group's candidates must fit a drained queue");
  __shared__ T sQv[QCAP][BM];
  __shared__ uint32_t sQj[QCAP][BM];
  int qn = 0;
  auto list_insert = [&](T sv, uint32_t jc) {
    // The new column comes after every listed one, so it goes behind the
    // values it equals: slot p takes slot p - 1 where the new value lands
    // before that, the new value where it lands between the two, and
    // otherwise stays.
    bool below = true;  // sv < lv[KL - 1], as the caller checked
#pragma unroll
    for (int p = KL - 1; p > 0; --p) {
      const bool below_prev = sv < lv[p - 1];
      lv[p] = below_prev ? lv[p - 1] : (below ? sv : lv[p]);
      lj[p] = below_prev ? lj[p - 1] : (below ? jc : lj[p]);
      below = below_prev;
    }
    lv[0] = below ? sv : lv[0];
    lj[0] = below ? jc : lj[0];
    thr = lv[KL - 1];
  };
  // Wave-uniform: every lane inserts its queued candidates in order.
  auto drain = [&]() {
    for (int q = 0; __any(q < qn); ++q) {
      if (q < qn) {
        const T v = sQv[q][tid];
        if (v < thr) list_insert(v, sQj[q][tid]);
      }
    }
    qn = 0;
  };

  for (int64_t j0 = jfirst; j0 < jlast; j0 += BN) {
    const int nb = (int)min((int64_t)BN, je - j0);
    const int cls = tile_class(mk, r0, r1, j0, j0 + nb - 1, rb, j0 / BN);
    if (cls == TILE_SKIP) continue;  // uniform over the workgroup
    const bool check = cls == TILE_CHECK;
    j0c = j0;
    __syncthreads();
    for (int e = tid; e < BN * DT; e += BM) {
      int jj = e / DT, d = e % DT;
      sY[jj][d] = (jj < nb && d < a.D) ? ldg<T>(bp.Y, (j0 + jj) * a.ldy + d) * pre_s : (T)0;
    }
    if constexpr (HAS_V) {
      for (int e = tid; e < BN * VW; e += BM) {
        int jj = e / VW, c = e % VW;
        sV[jj][c] = (jj < nb && c < a.C) ? ldg<T>(bp.V, (j0 + jj) * a.ldv + c) : (T)0;
      }
    }
    if constexpr (METRIC == M_COSINE) {
      for (int e = tid; e < BN; e += BM) sR[e] = e < nb ? ldg<T>(bp.ny, j0 + e) : (T)0;
    }
    if (check) {
      for (int e = tid; e < BN; e += BM) {
        sC[e] = (e < nb && (!mk.col || mk.col[j0 + e])) ? 1 : 0;
        sG[e] = (e < nb && mk.grow) ? mk.gcol[j0 + e] : 0;
      }
    }
    if (a.epi.any_col) {
      for (int e = tid; e < kMaxStages * BN; e += BM) {
        int st = e / BN, jj = e % BN;
        if (st < a.epi.n_stages && a.epi.st[st].col_vec) {
          bool ok = jj < nb;
          sQ[st][jj] = ok ? ldg<T>(epi_vec(a, a.epi.st[st].q_vec), j0 + jj) : (T)1;
          sO[st][jj] = ok ? ldg<T>(epi_vec(a, a.epi.st[st].o_vec), j0 + jj) : (T)0;
        }
      }
    }
    __syncthreads();
    if (!rv) continue;
    // A plain tile (full width, nothing masked, no diagonal to drop) runs at
    // a constant trip count with no per-column conditions; the others take
    // the same sweep with the conditions in.
    const bool plain = nb == BN && !check &&
                       !(CONS == C_LOGSUMEXP && a.exclude_self && j0 <= r1 && j0 + BN > r0);
    auto sweep = [&](auto plain_tag) {
      constexpr bool PLAIN = decltype(plain_tag)::value;
      const int n = PLAIN ? BN : nb;
      const bool chk = !PLAIN && check;
      // k = 1: the tile slot of the best column met in this tile (-1: none);
      // a constant slot number makes the select cheaper than a column index.
      int bl = -1;
      // One column at a time: unrolled deeply on plain tiles, where nothing
      // branches between columns.
      auto cols = [&](auto body) {
        if constexpr (PLAIN && HAS_V) {
#pragma unroll 4
          for (int jj = 0; jj < BN; ++jj) body(jj);
        } else if constexpr (PLAIN) {
#pragma unroll 8
          for (int jj = 0; jj < BN; ++jj) body(jj);
        } else {
          for (int jj = 0; jj < n; ++jj) body(jj);
        }
      };
      if constexpr (CONS == C_LOGSUMEXP || CONS == C_SOFTMAX) {
        // Pairs that carry no weight: the row's own column under
        // exclude_self, and masked pairs of a checked tile.
        auto dropped = [&](int jj) -> bool {
          if constexpr (PLAIN) return false;
          return (CONS == C_LOGSUMEXP && a.exclude_self && j0 + jj == i) || (chk && !kept(jj));
        };
        if (fast2) {
          // float, at most one row-only affine stage: scores are kept in
          // base 2 relative to a reference m2, s2 - m2 = (r_i log2e) f +
          // (p_i log2e - m2) in one FMA, and weighted 2^(s2 - m2) with the
          // hardware exponential. The reference moves only when a group's
          // maximum exceeds it by more than 8 (so weights stay <= 256); it
          // counts as 0 until the first finite score.
#pragma unroll 1
          for (int g = 0; g < n; g += G) {
            T sv[G];
            T gm = neg_inf<T>();
#pragma unroll
            for (int u = 0; u < G; ++u) {
              const int jj = g + u;
              T s = neg_inf<T>();
              if (PLAIN || jj < n) {
                s = fma(metric(jj), r2, q2);
                if (dropped(jj)) s = neg_inf<T>();
              }
              sv[u] = s;
              gm = max(gm, s);
            }
            const bool first = m == neg_inf<T>();
            if (gm > (first ? neg_inf<T>() : (T)8)) {
              const T alpha = first ? (T)0 : __builtin_amdgcn_exp2f(-gm);
              l *= alpha;
              if constexpr (CONS == C_SOFTMAX) {
#pragma unroll
                for (int c = 0; c < ACCN; ++c) acc[c] *= alpha;
              }
              m = (first ? (T)0 : m) + gm;
              q2 = p2 - m;
#pragma unroll
              for (int u = 0; u < G; ++u) sv[u] -= gm;
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
              const T p = __builtin_amdgcn_exp2f(sv[u]);
              l += p;
              if constexpr (CONS == C_SOFTMAX) {
#pragma unroll
                for (int c = 0; c < ACCN; ++c) acc[c] = fma(p, sV[g + u][c], acc[c]);
              }
            }
          }
          return;
        }
#pragma unroll 1
        for (int g = 0; g < n; g += G) {
          T sv[G];
          T gm = neg_inf<T>();
#pragma unroll
          for (int u = 0; u < G; ++u) {
            const int jj = g + u;
            T s = neg_inf<T>();
            if (PLAIN || jj < n) {
              s = apply_epi<T, BN>(a.epi, re, metric(jj), sQ, sO, jj);
              if (dropped(jj)) s = neg_inf<T>();
            }
            sv[u] = s;
            gm = max(gm, s);
          }
          if (gm > m) {
            const T alpha = dexp(m - gm);
            l *= alpha;
            if constexpr (CONS == C_SOFTMAX) {
#pragma unroll
              for (int c = 0; c < ACCN; ++c) acc[c] *= alpha;
            }
            m = gm;
          }
          if (m != neg_inf<T>()) {
#pragma unroll
            for (int u = 0; u < G; ++u) {
              const T p = dexp(sv[u] - m);
              l += p;
              if constexpr (CONS == C_SOFTMAX) {
#pragma unroll
                for (int c = 0; c < ACCN; ++c) acc[c] = fma(p, sV[g + u][c], acc[c]);
              }
            }
          }
        }
      } else {
        auto fold = [&](int jj, T s) {
          if constexpr (CONS == C_MATMUL) {
#pragma unroll
            for (int c = 0; c < ACCN; ++c) acc[c] = fma(s, sV[jj][c], acc[c]);
          } else if constexpr (CONS == C_DISPLACEMENT) {
#pragma unroll
            for (int d = 0; d < ACCN; ++d) acc[d] = fma(s, sY[jj][d], acc[d]);
            mass += s;
          }
        };
        // Top-k: columns reach a thread in increasing order, so a candidate
        // enters only when its signed value is strictly below the threshold.
        auto fold_topk = [&](int jj, T sv) {
          if constexpr (KL == 1) {
            const bool lt = sv < thr;
            thr = lt ? sv : thr;
            bl = lt ? jj : bl;
          } else {
            // One column: drain first if some lane's queue is full.
            const bool hit = sv < thr;
            if (__any(hit)) {
              if (__any(qn == QCAP)) drain();
              if (hit && sv < thr) {
                sQv[qn][tid] = sv;
                sQj[qn][tid] = (uint32_t)(j0 + jj);
                ++qn;
              }
            }
          }
        };
        // A group of G columns whose smallest value is below the threshold:
        // drain first if some lane could not queue the whole group.
        auto fold_group = [&](int g, const T (&sv)[G], T lo) {
          const bool hit = lo < thr;
          if (__any(hit)) {
            if (__any(qn > QCAP - G)) drain();
            if (hit) {
#pragma unroll
              for (int u = 0; u < G; ++u) {
                if (sv[u] < thr) {
                  sQv[qn][tid] = sv[u];
                  sQj[qn][tid] = (uint32_t)(j0 + g + u);
                  ++qn;
                }
              }
            }
          }
        };
        // With k > 1 and short rows a group of G columns is screened by its
        // smallest signed value first: most groups hold no candidate once the
        // list is full. Long rows amortise the per-column test already.
        auto topk_sweep = [&](auto score) {
          if constexpr (KL == 1 && PLAIN) {
            // Groups of G columns with a constant slot inside the group, so
            // that the select of the best slot takes an inline constant.
#pragma unroll 1
            for (int g = 0; g < BN; g += G) {
              int bu = -1;
#pragma unroll
              for (int u = 0; u < G; ++u) {
                const T sv = score(g + u);
                const bool lt = sv < thr;
                thr = lt ? sv : thr;
                bu = lt ? u : bu;
              }
              bl = bu >= 0 ? g + bu : bl;
            }
          } else if constexpr (KL == 1 || DT > 4) {
            cols([&](int jj) { fold_topk(jj, score(jj)); });
          } else {
#pragma unroll 1
            for (int g = 0; g < n; g += G) {
              T sv[G];
              T lo = (T)__builtin_huge_val();
#pragma unroll
              for (int u = 0; u < G; ++u) {
                sv[u] = (PLAIN || g + u < n) ? score(g + u) : (T)__builtin_huge_val();
                lo = min(lo, sv[u]);
              }
              fold_group(g, sv, lo);
            }
          }
        };
        // Checked tiles drop masked pairs: no weight in a sum, +inf (never a
        // candidate) in the signed top-k orientation. The stage loop runs
        // only when the expression has score arithmetic (a uniform branch).
        if (chk) {
          const T sg = a.largest ? (T)-1 : (T)1;
          for (int jj = 0; jj < n; ++jj) {
            const T sc = apply_epi<T, BN>(a.epi, re, metric(jj), sQ, sO, jj);
            const bool kp = kept(jj);
            if constexpr (CONS == C_TOPK) fold_topk(jj, kp ? sg * sc : (T)__builtin_huge_val());
            else fold(jj, kp ? sc : (T)0);
          }
        } else if constexpr (CONS == C_TOPK) {
          if (a.epi.n_stages == 0) {
            if (a.largest) topk_sweep([&](int jj) { return -metric(jj); });
            else topk_sweep([&](int jj) { return metric(jj); });
          } else {
            const T sg = a.largest ? (T)-1 : (T)1;
            topk_sweep([&](int jj) { return sg * apply_epi<T, BN>(a.epi, re, metric(jj), sQ, sO, jj); });
          }
        } else if (a.epi.n_stages == 0) {
          cols([&](int jj) { fold(jj, metric(jj)); });
        } else {
          cols([&](int jj) { fold(jj, apply_epi<T, BN>(a.epi, re, metric(jj), sQ, sO, jj)); });
        }
        if constexpr (CONS == C_TOPK && KL == 1) {
          if (bl >= 0) best_j = (uint32_t)(j0 + bl);
        }
      }
    };
    // Only narrow rows and value widths take the plain variant: it lets the
    // compiler hoist a whole group's LDS reads, which wide ones cannot hold.
    if constexpr (DT <= 4 && VW <= 4) {
      if (plain) sweep(Bool<true>{});
      else sweep(Bool<false>{});
    } else {
      sweep(Bool<false>{});
    }
  }
  if constexpr (QUEUE) drain();
  if (!rv) return;
  if (fast2 && m != neg_inf<T>()) m *= (T)kLn2;  // back to natural units
  if (!rkeep) {  // a masked row: the empty-row result
#pragma unroll
    for (int c = 0; c < ACCN; ++c) acc[c] = 0;
    mass = 0;
    m = neg_inf<T>();
    l = 0;
#pragma unroll
    for (int p = 0; p < KL; ++p) lj[p] = ~0u;
    best_j = ~0u;
  }

  const bool fin = a.n_split == 1;
  const int64_t prow = (int64_t)sp * a.N + i;  // partial row
  if constexpr (CONS == C_MATMUL) {
    T *o = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow * a.C;
#pragma unroll
    for (int c = 0; c < ACCN; ++c)
      if (c < a.C) o[c] = acc[c];
  } else if constexpr (CONS == C_DISPLACEMENT) {
    T *o = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow * a.D;
#pragma unroll
    for (int d = 0; d < ACCN; ++d)
      if (d < a.D) o[d] = acc[d] - x[d] * mass;
  } else if constexpr (CONS == C_LOGSUMEXP) {
    if (fin) {
      static_cast<T *>(bp.out)[i] = (l > (T)0) ? m + dlog(l) : neg_inf<T>();
    } else {
      T *o = static_cast<T *>(bp.partial) + prow * 2;
      o[0] = m;
      o[1] = l;
    }
  } else if constexpr (CONS == C_SOFTMAX) {
    if (fin && bp.lse_out) static_cast<T *>(bp.lse_out)[i] = (l > (T)0) ? m + dlog(l) : neg_inf<T>();
    if (fin) {
      T *o = static_cast<T *>(bp.out) + i * a.ldo;
      const T inv = (l > (T)0) ? (T)1 / l : (T)0;
#pragma unroll
      for (int c = 0; c < ACCN; ++c)
        if (c < a.C) o[c] = acc[c] * inv;
    } else {
      T *o = static_cast<T *>(bp.partial) + prow * (a.C + 2);
      o[0] = m;
      o[1] = l;
#pragma unroll
      for (int c = 0; c < ACCN; ++c)
        if (c < a.C) o[2 + c] = acc[c];
    }
  } else if constexpr (CONS == C_TOPK) {
    if constexpr (KL == 1) {
      lv[0] = thr;
      lj[0] = best_j;
    }
    Key<T> list[KL];
#pragma unroll
    for (int p = 0; p < KL; ++p)
      list[p] = lj[p] == ~0u ? Key<T>::sentinel() : Key<T>::make(a.largest ? -lv[p] : lv[p], lj[p], a.largest);
    if (fin) {
      T *v = static_cast<T *>(bp.out) + i * a.k;
      int64_t *ix = bp.idx + i * a.k;
#pragma unroll
      for (int p = 0; p < KL; ++p)
        if (p < a.k) {
          v[p] = list[p].value(a.largest);
          ix[p] = list[p].out_index();
        }
    } else {
#pragma unroll
      for (int p = 0; p < KL; ++p)
        if (p < a.k) list[p].store(bp.partial, prow * a.k + p);
    }
  }
}

// The plain float kernel product (no score arithmetic, no masks, D <= 4,
// C <= 4) with R rows per thread: every broadcast read of a column, which
// costs the LDS its full width, serves R rows' pairs. Thread t owns rows
// t, t + 256, ... of an R * 256-row block. Column tiles of 256 (one column
// per thread) are loaded one tile ahead into registers and double-buffered
// in LDS, one barrier per tile. Columns past the split's end are staged as
// zeros, so their value rows add nothing.
//
// rbf scores are exponentials of base 2 of points pre-scaled by
// sqrt(gamma log2 e), so exp(-gamma |x - y|^2) = 2^-|x~ - y~|^2. Where every
// row of a wave and every column of the tile has |x~|^2, |y~|^2 <= 64, the
// exponent is formed by the norm expansion with the row's own term left
// out, t = 2 x~.y~ - |y~|^2 (three FMAs from a staged (y~, -|y~|^2)), and
// the row factor 2^-|x~|^2 multiplies the finished sums; t <= |x~|^2 <= 64,
// so no term overflows. Elsewhere (points far from the origin, where the
// expansion would cancel) the pair takes the direct form, its exponent
// started at the row's deferred |x~|^2 when the wave defers it (else at 0),
// so identical points still score exactly 1 there.
constexpr float kExpansionBound = 64.f;

// Waves per SIMD each product kernel is held to: what its registers allow,
// so that the scheduler does not trade occupancy for a deeper schedule.
constexpr int prod_waves(int metric, int dt) { return metric == M_RBF ? (dt == 3 ? 5 : 4) : (dt == 3 ? 8 : 7); }

template <int METRIC, int DT, int R>
__global__ __launch_bounds__(kValuBM) __attribute__((amdgpu_waves_per_eu(prod_waves(METRIC, DT)))) void valu_prod_rn(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  constexpr int BN = kValuBM;  // columns per tile: one staged per thread
  static_assert(DT == 3 || DT == 4, "narrow points only");
  constexpr bool RBF = METRIC == M_RBF;
  __shared__ float4 sY[2][BN];  // (y0, y1, y2, -|y~|^2) for DT = 3, else (y0..y3)
  __shared__ float sW[2][DT == 4 ? BN : 1];  // -|y~|^2 for DT = 4
  __shared__ float4 sV[2][BN];
  __shared__ int sFar[2];  // tile index whose staging met a column with |y~|^2 > bound
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb;
  const int sp = blockIdx.x / a.n_rb;
  const int64_t jb = wave_uniform((int64_t)sp * a.split_cols);
  const int64_t je = wave_uniform(min(a.M, jb + a.split_cols));
  const int n_tiles = (int)((je - jb + BN - 1) / BN);
  const float pre_s = RBF ? (float)sqrt(a.gamma * kLog2e) : 1.f;

  // Row operand: 2 x~ for rbf (the expansion's factor; x~ = half of it,
  // exactly), else x itself. One copy keeps the rbf kernel within five waves
  // per SIMD for three features (four for four).
  int64_t i[R];
  float xr[R][DT], acc[R][4], x0[R];
  bool near_all = true;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    i[u] = (int64_t)rb * (R * BN) + u * BN + tid;
    const bool rv = i[u] < a.N;
    float n2 = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const float xv = (rv && d < a.D) ? ldg<float>(bp.X, i[u] * a.ldx + d) * pre_s : 0.f;
      xr[u][d] = RBF ? 2.f * xv : xv;
      n2 = fmaf(xv, xv, n2);
    }
    x0[u] = n2;  // deferred row term |x~|^2 (rbf)
    near_all = near_all && n2 <= kExpansionBound;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[u][c] = 0.f;
  }
  // The wave defers the row factor only if no row can overflow.
  const bool defer = RBF && __all(near_all);
  if (!defer) {
#pragma unroll
    for (int u = 0; u < R; ++u) x0[u] = 0.f;
  }

  // Staging registers: this thread's column of the next tile.
  float ry[DT], rv4[4];
  auto fetch = [&](int t) {
    const int64_t j = jb + (int64_t)t * BN + tid;
    const bool cv = j < je;
#pragma unroll
    for (int d = 0; d < DT; ++d) ry[d] = (cv && d < a.D) ? ldg<float>(bp.Y, j * a.ldy + d) : 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) rv4[c] = (cv && c < a.C) ? ldg<float>(bp.V, j * a.ldv + c) : 0.f;
  };
  auto stage = [&](int t) {
    const int b = t & 1;
    float y[4] = {0.f, 0.f, 0.f, 0.f}, n2 = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      y[d] = ry[d] * pre_s;
      n2 = fmaf(y[d], y[d], n2);
    }
    if constexpr (DT == 3) y[3] = -n2;
    else sW[b][tid] = -n2;
    sY[b][tid] = make_float4(y[0], y[1], y[2], y[3]);
    sV[b][tid] = make_float4(rv4[0], rv4[1], rv4[2], rv4[3]);
    if (RBF && n2 > kExpansionBound) sFar[b] = t;
  };

  if (tid < 2) sFar[tid] = -1;
  __syncthreads();
  if (n_tiles > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int b = t & 1;
    if (t + 1 < n_tiles) fetch(t + 1);
    const float4 *Yb = sY[b];
    const float4 *Vb = sV[b];
    if (RBF && defer && sFar[b] != t) {
      // Norm expansion, row factor deferred.
#pragma unroll 4
      for (int jj = 0; jj < BN; ++jj) {
        const float4 y = Yb[jj];
        const float4 v = Vb[jj];
        const float w = DT == 3 ? y.w : sW[b][jj];
#pragma unroll
        for (int u = 0; u < R; ++u) {
          float e = fmaf(xr[u][0], y.x, w);
          e = fmaf(xr[u][1], y.y, e);
          e = fmaf(xr[u][2], y.z, e);
          if constexpr (DT == 4) e = fmaf(xr[u][3], y.w, e);
          const float k = __builtin_amdgcn_exp2f(e);
          acc[u][0] = fmaf(k, v.x, acc[u][0]);
          acc[u][1] = fmaf(k, v.y, acc[u][1]);
          acc[u][2] = fmaf(k, v.z, acc[u][2]);
          acc[u][3] = fmaf(k, v.w, acc[u][3]);
        }
      }
    } else {
      // Direct form.
#pragma unroll 2
      for (int jj = 0; jj < BN; ++jj) {
        const float4 y = Yb[jj];
        const float4 v = Vb[jj];
        const float yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int u = 0; u < R; ++u) {
          float sc;
          if constexpr (METRIC == M_LINEAR) {
            sc = xr[u][0] * yy[0];
#pragma unroll
            for (int d = 1; d < DT; ++d) sc = fmaf(xr[u][d], yy[d], sc);
          } else {
            float e = x0[u];
#pragma unroll
            for (int d = 0; d < DT; ++d) {
              const float df = RBF ? fmaf(xr[u][d], 0.5f, -yy[d]) : xr[u][d] - yy[d];
              e = fmaf(-df, df, e);
            }
            sc = RBF ? __builtin_amdgcn_exp2f(e) : -e;
          }
          acc[u][0] = fmaf(sc, v.x, acc[u][0]);
          acc[u][1] = fmaf(sc, v.y, acc[u][1]);
          acc[u][2] = fmaf(sc, v.z, acc[u][2]);
          acc[u][3] = fmaf(sc, v.w, acc[u][3]);
        }
      }
    }
    if (t + 1 < n_tiles) stage(t + 1);
    __syncthreads();
  }
  const bool fin = a.n_split == 1;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (i[u] >= a.N) continue;
    const float f = (RBF && defer) ? __builtin_amdgcn_exp2f(-x0[u]) : 1.f;
    float *o = fin ? static_cast<float *>(bp.out) + i[u] * a.ldo
                   : static_cast<float *>(bp.partial) + ((int64_t)sp * a.N + i[u]) * a.C;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < a.C) o[c] = acc[u][c] * f;
  }
}

// The plain float row minimum (or maximum) with its column, two rows per
// thread (rows i and i + 256 of a 512-row block, 64-column tiles). Columns
// reach a thread in increasing order and
// a candidate must be strictly better, so the lowest index wins a tie.
template <int METRIC, int DT, bool LARGEST>
__device__ __forceinline__ void r2_min_tile(const float (&x)[2][DT], const float (*sY)[DT], int n, float neg_gamma,
                                            float (&thr)[2], int (&bl)[2]) {
  constexpr bool PRE = METRIC == M_RBF;
  auto body = [&](int jj) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float sc = valu_metric<METRIC, float, DT, PRE>(x[u], sY[jj], neg_gamma);
      const float sv = LARGEST ? -sc : sc;
      const bool lt = sv < thr[u];
      thr[u] = lt ? sv : thr[u];
      bl[u] = lt ? jj : bl[u];
    }
  };
  if (n == kValuBN) {
#pragma unroll 8
    for (int jj = 0; jj < kValuBN; ++jj) body(jj);
  } else {
    for (int jj = 0; jj < n; ++jj) body(jj);
  }
}

// Three-feature squared distances by the norm expansion with the row's own
// term left out: a staged column holds (y, |y|^2), a row holds -2x, and
// three FMAs give u = |y|^2 - 2 x.y. fl(|x|^2 + u) is monotone in u, so the
// row's extreme u, plus |x|^2 and clamped at 0, is its extreme distance;
// a tie the final rounding creates is within the pair's rounding error.
template <bool LARGEST>
__device__ __forceinline__ void r2_min_tile_exp(const float (&xm)[2][3], const float (*sY)[4], int n,
                                                float (&thr)[2], int (&bl)[2]) {
  auto body = [&](int jj) {
    const float4 y = *reinterpret_cast<const float4 *>(sY[jj]);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float sc = fma(xm[u][0], y.x, fma(xm[u][1], y.y, fma(xm[u][2], y.z, y.w)));
      const float sv = LARGEST ? -sc : sc;
      const bool lt = sv < thr[u];
      thr[u] = lt ? sv : thr[u];
      bl[u] = lt ? jj : bl[u];
    }
  };
  if (n == kValuBN) {
#pragma unroll 8
    for (int jj = 0; jj < kValuBN; ++jj) body(jj);
  } else {
    for (int jj = 0; jj < n; ++jj) body(jj);
  }
}

template <int METRIC, int DT>
__global__ __launch_bounds__(kValuBM) __attribute__((amdgpu_waves_per_eu(8))) void valu_tile_r2_min(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  constexpr int BN = kValuBN, R = 2;
  // Three-feature squared distances take the expansion (columns staged with
  // their norms); other shapes and metrics are evaluated directly.
  constexpr bool EXP = METRIC == M_SQEUCLIDEAN && DT == 3;
  constexpr int SW = EXP ? 4 : DT;
  __shared__ __attribute__((aligned(16))) float sY[BN][SW];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb;
  const int sp = blockIdx.x / a.n_rb;
  const int64_t jb = wave_uniform((int64_t)sp * a.split_cols);
  const int64_t je = wave_uniform(min(a.M, jb + a.split_cols));
  constexpr bool PRE = METRIC == M_RBF;
  const float pre_s = PRE ? (float)sqrt(a.gamma * kLog2e) : 1.f;
  const float neg_gamma = (float)(-a.gamma * kLog2e);
  int64_t i[R];
  bool rv[R];
  float x[R][DT], thr[R], nx[R];
  uint32_t bj[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    i[u] = (int64_t)rb * (R * kValuBM) + u * kValuBM + tid;
    rv[u] = i[u] < a.N;
#pragma unroll
    for (int d = 0; d < DT; ++d) x[u][d] = (rv[u] && d < a.D) ? ldg<float>(bp.X, i[u] * a.ldx + d) * pre_s : 0.f;
    thr[u] = __builtin_huge_valf();
    bj[u] = ~0u;
    nx[u] = 0.f;
    if constexpr (EXP) {
      nx[u] = fma(x[u][0], x[u][0], fma(x[u][1], x[u][1], x[u][2] * x[u][2]));
#pragma unroll
      for (int d = 0; d < DT; ++d) x[u][d] *= -2.f;
    }
  }
  for (int64_t j0 = jb; j0 < je; j0 += BN) {
    const int nb = (int)min((int64_t)BN, je - j0);
    __syncthreads();
    if constexpr (EXP) {
      if (tid < BN) {
        float y[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) y[d] = (tid < nb && d < a.D) ? ldg<float>(bp.Y, (j0 + tid) * a.ldy + d) : 0.f;
        *reinterpret_cast<float4 *>(sY[tid]) =
            make_float4(y[0], y[1], y[2], fma(y[0], y[0], fma(y[1], y[1], y[2] * y[2])));
      }
    } else {
      for (int e = tid; e < BN * DT; e += kValuBM) {
        const int jj = e / DT, d = e % DT;
        sY[jj][d] = (jj < nb && d < a.D) ? ldg<float>(bp.Y, (j0 + jj) * a.ldy + d) * pre_s : 0.f;
      }
    }
    __syncthreads();
    int bl[R] = {-1, -1};  // tile slot of each row's best column met in this tile
    if constexpr (EXP) {
      if (a.largest) r2_min_tile_exp<true>(x, sY, nb, thr, bl);
      else r2_min_tile_exp<false>(x, sY, nb, thr, bl);
    } else {
      if (a.largest) r2_min_tile<METRIC, DT, true>(x, sY, nb, neg_gamma, thr, bl);
      else r2_min_tile<METRIC, DT, false>(x, sY, nb, neg_gamma, thr, bl);
    }
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (bl[u] >= 0) bj[u] = (uint32_t)(j0 + bl[u]);
  }
  const bool fin = a.n_split == 1;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (!rv[u]) continue;
    float best = a.largest ? -thr[u] : thr[u];
    if constexpr (EXP) best = max(nx[u] + best, 0.f);
    const Key<float> key = bj[u] == ~0u ? Key<float>::sentinel() : Key<float>::make(best, bj[u], a.largest);
    if (fin) {
      static_cast<float *>(bp.out)[i[u] * a.k] = key.value(a.largest);
      bp.idx[i[u] * a.k] = key.out_index();
    } else {
      key.store(bp.partial, ((int64_t)sp * a.N + i[u]) * a.k);
    }
  }
}

// The float row log-sum-exp of narrow points under at most one row-only
// affine stage, two rows per thread. Scores are kept in base 2 relative to
// a reference m (moved only when a group of 8 columns exceeds it by more
// than 8, so weights stay <= 256), as the one-row engine does. Tiles that
// meet a row's own column under exclude_self check every pair.
template <int METRIC, int DT, bool CHECK>
__device__ __forceinline__ void r2_lse_tile(const float (&x)[2][DT], const float (*sY)[DT], int n, float neg_gamma,
                                            const float (&r2)[2], const float (&p2)[2], float (&q2)[2],
                                            float (&m)[2], float (&l)[2], int64_t j0, const int64_t (&i)[2],
                                            bool excl) {
  constexpr bool PRE = METRIC == M_RBF;
  constexpr int G = 8;
  const int ng = CHECK ? n : kValuBN;
#pragma unroll 1
  for (int g = 0; g < ng; g += G) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float sv[G];
      float gm = -__builtin_huge_valf();
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int jj = g + k;
        float sc = fma(valu_metric<METRIC, float, DT, PRE>(x[u], sY[jj], neg_gamma), r2[u], q2[u]);
        if (CHECK && (jj >= n || (excl && j0 + jj == i[u]))) sc = -__builtin_huge_valf();
        sv[k] = sc;
        gm = fmaxf(gm, sc);
      }
      const bool first = m[u] == -__builtin_huge_valf();
      if (gm > (first ? -__builtin_huge_valf() : 8.f)) {
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-gm);
        l[u] *= alpha;
        m[u] = (first ? 0.f : m[u]) + gm;
        q2[u] = p2[u] - m[u];
#pragma unroll
        for (int k = 0; k < G; ++k) sv[k] -= gm;
      }
#pragma unroll
      for (int k = 0; k < G; ++k) l[u] += __builtin_amdgcn_exp2f(sv[k]);
    }
  }
}

template <int METRIC, int DT>
__global__ __launch_bounds__(kValuBM) void valu_tile_r2_lse(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  constexpr int BN = kValuBN, R = 2;
  __shared__ float sY[BN][DT];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb;
  const int sp = blockIdx.x / a.n_rb;
  const int64_t jb = wave_uniform((int64_t)sp * a.split_cols);
  const int64_t je = wave_uniform(min(a.M, jb + a.split_cols));
  const int64_t r0 = (int64_t)rb * (R * kValuBM), r1 = min(a.N, r0 + R * kValuBM) - 1;
  constexpr bool PRE = METRIC == M_RBF;
  const float pre_s = PRE ? (float)sqrt(a.gamma * kLog2e) : 1.f;
  const float neg_gamma = (float)(-a.gamma * kLog2e);
  int64_t i[R];
  bool rv[R];
  float x[R][DT], r2[R], p2[R], q2[R], m[R], l[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    i[u] = r0 + u * kValuBM + tid;
    rv[u] = i[u] < a.N;
#pragma unroll
    for (int d = 0; d < DT; ++d) x[u][d] = (rv[u] && d < a.D) ? ldg<float>(bp.X, i[u] * a.ldx + d) * pre_s : 0.f;
    float r = 1.f, p = 0.f;
    if (a.epi.n_stages == 1) {
      const Stage &st = a.epi.st[0];
      if (st.row_vec) {
        if (rv[u]) {
          r = ldg<float>(epi_vec(a, st.r_vec), i[u]);
          p = ldg<float>(epi_vec(a, st.p_vec), i[u]);
        }
      } else {
        r = (float)st.r_scalar;
        p = (float)st.p_scalar;
      }
    }
    r2[u] = kLog2e_f * r;
    p2[u] = kLog2e_f * p;
    q2[u] = p2[u];
    m[u] = -__builtin_huge_valf();
    l[u] = 0.f;
  }
  const bool excl = a.exclude_self != 0;
  for (int64_t j0 = jb; j0 < je; j0 += BN) {
    const int nb = (int)min((int64_t)BN, je - j0);
    __syncthreads();
    for (int e = tid; e < BN * DT; e += kValuBM) {
      const int jj = e / DT, d = e % DT;
      sY[jj][d] = (jj < nb && d < a.D) ? ldg<float>(bp.Y, (j0 + jj) * a.ldy + d) * pre_s : 0.f;
    }
    __syncthreads();
    const bool check = nb < BN || (excl && j0 <= r1 && j0 + BN > r0);  // uniform over the workgroup
    if (check) r2_lse_tile<METRIC, DT, true>(x, sY, nb, neg_gamma, r2, p2, q2, m, l, j0, i, excl);
    else r2_lse_tile<METRIC, DT, false>(x, sY, nb, neg_gamma, r2, p2, q2, m, l, j0, i, excl);
  }
  const bool fin = a.n_split == 1;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (!rv[u]) continue;
    const float mn = m[u] == -__builtin_huge_valf() ? m[u] : m[u] * kLn2_f;  // back to natural units
    if (fin) {
      static_cast<float *>(bp.out)[i[u]] = l[u] > 0.f ? mn + dlog(l[u]) : -__builtin_huge_valf();
    } else {
      float *o = static_cast<float *>(bp.partial) + ((int64_t)sp * a.N + i[u]) * 2;
      o[0] = mn;
      o[1] = l[u];
    }
  }
}

// The float row log-sum-exp of narrow points, linear or squared euclidean,
// under at most one row-only affine stage s = r_i f + p_i: four rows per
// thread and 256-column tiles loaded one tile ahead, as the product above.
// In base 2 and relative to the row's reference m,
//   s2 - m = C_i + B_i |y|^2 + A_i . y,
// with B_i = r_i log2 e, A_i = -2 B_i x_i and C_i = B_i |x_i|^2 + p_i log2 e
// - m for the squared distance (its norm expansion: four FMAs a pair at
// three features), and A_i = B_i x_i, C_i = p_i log2 e - m, no |y|^2 term,
// for the dot product. The reference moves only when a group of 8 columns
// exceeds it by more than 8 (weights stay <= 256) and counts as 0 until the
// first finite score, as in the one-row engine. The ragged last tile and
// tiles that meet a row's own column under exclude_self check every pair.

template <int METRIC, int DT, int R>
__global__ __launch_bounds__(kValuBM) void valu_lse_rn(const TileArgs a) {
  static_assert(METRIC == M_LINEAR || METRIC == M_SQEUCLIDEAN, "dot product or squared distance");
  static_assert(DT == 3 || DT == 4, "narrow points only");
  const BatchPtrs bp = batch_ptrs(a);
  constexpr int BN = kValuBM, G = 4;
  constexpr bool SQ = METRIC == M_SQEUCLIDEAN;
  __shared__ float4 sY[2][BN];                // (y0, y1, y2, |y|^2) for DT = 3, else (y0..y3)
  __shared__ float sW[2][DT == 4 ? BN : 1];   // |y|^2 for DT = 4
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.n_rb;
  const int sp = blockIdx.x / a.n_rb;
  const int64_t jb = wave_uniform((int64_t)sp * a.split_cols);
  const int64_t je = wave_uniform(min(a.M, jb + a.split_cols));
  const int n_tiles = (int)((je - jb + BN - 1) / BN);
  const int64_t r0 = (int64_t)rb * (R * BN), r1 = min(a.N, r0 + R * BN) - 1;

  float A[R][DT], B[R], P[R], C[R], m[R], l[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int64_t i = r0 + u * BN + tid;
    const bool rv = i < a.N;
    float r = 1.f, p = 0.f;
    if (a.epi.n_stages == 1) {
      const Stage &st = a.epi.st[0];
      if (st.row_vec) {
        if (rv) {
          r = ldg<float>(epi_vec(a, st.r_vec), i);
          p = ldg<float>(epi_vec(a, st.p_vec), i);
        }
      } else {
        r = (float)st.r_scalar;
        p = (float)st.p_scalar;
      }
    }
    if (!rv) r = 0.f;  // rows past the end score 0 everywhere
    B[u] = kLog2e_f * r;
    float n2 = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const float xv = (rv && d < a.D) ? ldg<float>(bp.X, i * a.ldx + d) : 0.f;
      A[u][d] = (SQ ? -2.f * B[u] : B[u]) * xv;
      n2 = fmaf(xv, xv, n2);
    }
    P[u] = SQ ? fmaf(B[u], n2, kLog2e_f * p) : kLog2e_f * p;
    C[u] = P[u];
    m[u] = -__builtin_huge_valf();
    l[u] = 0.f;
  }

  float ry[DT];
  auto fetch = [&](int t) {
    const int64_t j = jb + (int64_t)t * BN + tid;
    const bool cv = j < je;
#pragma unroll
    for (int d = 0; d < DT; ++d) ry[d] = (cv && d < a.D) ? ldg<float>(bp.Y, j * a.ldy + d) : 0.f;
  };
  auto stage = [&](int t) {
    const int b = t & 1;
    float y[4] = {0.f, 0.f, 0.f, 0.f}, n2 = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      y[d] = ry[d];
      n2 = fmaf(y[d], y[d], n2);
    }
    if constexpr (DT == 3) y[3] = n2;
    else sW[b][tid] = n2;
    sY[b][tid] = make_float4(y[0], y[1], y[2], y[3]);
  };

  // One tile of columns j0 + [0, n) from buffer b.
  auto sweep = [&](auto check_tag, int b, int64_t j0, int n) {
    constexpr bool CHECK = decltype(check_tag)::value;
    const float4 *Yb = sY[b];
    const bool excl = a.exclude_self != 0;
    int own[R];  // the row's own column as a tile slot (outside [0, BN) if not here)
#pragma unroll
    for (int u = 0; u < R; ++u) own[u] = (int)(r0 + u * BN + tid - j0);
#pragma unroll 1
    for (int g = 0; g < BN; g += G) {
      if (CHECK && g >= n) break;
      float4 y[G];
      float w[G];
#pragma unroll
      for (int k = 0; k < G; ++k) {
        y[k] = Yb[g + k];
        w[k] = DT == 3 ? y[k].w : sW[b][g + k];
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        float sv[G];
        float gm = -__builtin_huge_valf();
#pragma unroll
        for (int k = 0; k < G; ++k) {
          float e = SQ ? fmaf(B[u], w[k], C[u]) : C[u];
          e = fmaf(A[u][0], y[k].x, e);
          e = fmaf(A[u][1], y[k].y, e);
          e = fmaf(A[u][2], y[k].z, e);
          if constexpr (DT == 4) e = fmaf(A[u][3], y[k].w, e);
          if (CHECK && (g + k >= n || (excl && g + k == own[u]))) e = -__builtin_huge_valf();
          sv[k] = e;
          gm = fmaxf(gm, e);
        }
        const bool first = m[u] == -__builtin_huge_valf();
        if (gm > (first ? -__builtin_huge_valf() : 8.f)) {
          const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-gm);
          l[u] *= alpha;
          m[u] = (first ? 0.f : m[u]) + gm;
          C[u] = P[u] - m[u];
#pragma unroll
          for (int k = 0; k < G; ++k) sv[k] -= gm;
        }
#pragma unroll
        for (int k = 0; k < G; ++k) l[u] += __builtin_amdgcn_exp2f(sv[k]);
      }
    }
  };

  if (n_tiles > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int b = t & 1;
    if (t + 1 < n_tiles) fetch(t + 1);
    const int64_t j0 = jb + (int64_t)t * BN;
    const int nb = (int)min((int64_t)BN, je - j0);
    const bool check = nb < BN || (a.exclude_self && j0 <= r1 && j0 + BN > r0);  // uniform
    if (check) sweep(Bool<true>{}, b, j0, nb);
    else sweep(Bool<false>{}, b, j0, nb);
    if (t + 1 < n_tiles) stage(t + 1);
    __syncthreads();
  }
  const bool fin = a.n_split == 1;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int64_t i = r0 + u * BN + tid;
    if (i >= a.N) continue;
    const float mn = m[u] == -__builtin_huge_valf() ? m[u] : m[u] * kLn2_f;  // back to natural units
    if (fin) {
      static_cast<float *>(bp.out)[i] = l[u] > 0.f ? mn + dlog(l[u]) : -__builtin_huge_valf();
    } else {
      float *o = static_cast<float *>(bp.partial) + ((int64_t)sp * a.N + i) * 2;
      o[0] = mn;
      o[1] = l[u];
    }
  }
}

template <class T, int METRIC, int CONS, int DT, int VT>
hipError_t launch_valu_kernel(const TileArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.n_rb * a.n_split), 1, (unsigned)a.bat.n), block(kValuBM);
  hipLaunchKernelGGL((valu_tile<T, METRIC, CONS, DT, VT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class T, int METRIC, int CONS, int DT>
hipError_t valu_by_vt(int vt, const TileArgs &a, hipStream_t s) {
  if constexpr (CONS == C_MATMUL || CONS == C_SOFTMAX) {
    if (vt == 4) return launch_valu_kernel<T, METRIC, CONS, DT, 4>(a, s);
    if (vt == 16) return launch_valu_kernel<T, METRIC, CONS, DT, 16>(a, s);
    if (vt == 64) return launch_valu_kernel<T, METRIC, CONS, DT, 64>(a, s);
  } else if constexpr (CONS == C_TOPK) {
    if (vt == 1) return launch_valu_kernel<T, METRIC, CONS, DT, 1>(a, s);
    if (vt == 8) return launch_valu_kernel<T, METRIC, CONS, DT, 8>(a, s);
    if (vt == 16) return launch_valu_kernel<T, METRIC, CONS, DT, 16>(a, s);
    if (vt == 64) return launch_valu_kernel<T, METRIC, CONS, DT, 64>(a, s);
  } else {
    return launch_valu_kernel<T, METRIC, CONS, DT, 1>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC, int DT>
hipError_t valu_by_consumer(int consumer, int vt, const TileArgs &a, hipStream_t s) {
  switch (consumer) {
    case C_MATMUL: return valu_by_vt<T, METRIC, C_MATMUL, DT>(vt, a, s);
    case C_DISPLACEMENT: return valu_by_vt<T, METRIC, C_DISPLACEMENT, DT>(vt, a, s);
    case C_LOGSUMEXP: return valu_by_vt<T, METRIC, C_LOGSUMEXP, DT>(vt, a, s);
    case C_SOFTMAX: return valu_by_vt<T, METRIC, C_SOFTMAX, DT>(vt, a, s);
    case C_TOPK: return valu_by_vt<T, METRIC, C_TOPK, DT>(vt, a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC>
hipError_t valu_launch_metric(int consumer, const ValuConfig &cfg, const TileArgs &a, hipStream_t s) {
  if constexpr (sizeof(T) == 4 && METRIC != M_COSINE) {
    if (consumer == C_MATMUL && cfg.rows == kProdRows) {
      if ((cfg.dtile != 3 && cfg.dtile != 4) || cfg.vtile != 4) return hipErrorInvalidValue;
      dim3 grid((unsigned)(a.n_rb * a.n_split), 1, (unsigned)a.bat.n), block(kValuBM);
      if (cfg.dtile == 3) hipLaunchKernelGGL((valu_prod_rn<METRIC, 3, kProdRows>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((valu_prod_rn<METRIC, 4, kProdRows>), grid, block, 0, s, a);
      return hipGetLastError();
    }
    if constexpr (METRIC != M_RBF) {
      if (consumer == C_LOGSUMEXP && cfg.rows == kProdRows) {
        if (cfg.dtile != 3 && cfg.dtile != 4) return hipErrorInvalidValue;
        dim3 grid((unsigned)(a.n_rb * a.n_split), 1, (unsigned)a.bat.n), block(kValuBM);
        if (cfg.dtile == 3) hipLaunchKernelGGL((valu_lse_rn<METRIC, 3, kProdRows>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((valu_lse_rn<METRIC, 4, kProdRows>), grid, block, 0, s, a);
        return hipGetLastError();
      }
    }
    if (cfg.rows == 2) {
      if (cfg.dtile != 3 && cfg.dtile != 4) return hipErrorInvalidValue;
      dim3 grid((unsigned)(a.n_rb * a.n_split), 1, (unsigned)a.bat.n), block(kValuBM);
      if (consumer == C_LOGSUMEXP) {
        if (cfg.dtile == 3) hipLaunchKernelGGL((valu_tile_r2_lse<METRIC, 3>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((valu_tile_r2_lse<METRIC, 4>), grid, block, 0, s, a);
      } else if (consumer == C_TOPK && cfg.vtile == 1 && a.k == 1) {
        if (cfg.dtile == 3) hipLaunchKernelGGL((valu_tile_r2_min<METRIC, 3>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((valu_tile_r2_min<METRIC, 4>), grid, block, 0, s, a);
      } else {
        return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
  }
  if (cfg.rows != 1) return hipErrorInvalidValue;
  switch (cfg.dtile) {
    case 3: return valu_by_consumer<T, METRIC, 3>(consumer, cfg.vtile, a, s);
    case 4: return valu_by_consumer<T, METRIC, 4>(consumer, cfg.vtile, a, s);
    case 16: return valu_by_consumer<T, METRIC, 16>(consumer, cfg.vtile, a, s);
    case 64: return valu_by_consumer<T, METRIC, 64>(consumer, cfg.vtile, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pw
