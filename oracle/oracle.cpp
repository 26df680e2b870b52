// CPU oracle for lazily evaluated pairwise scores.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
// this file; only the test suite, the smoke check and the CPU-baseline leg of
// the benchmark do. It shares no code, header or constant with the GPU library.
//
// What it computes (torchpairwise guide "Using Torchpairwise in Models"):
//   * a pairwise score s_ij = f(x_i, y_j) for the built-in metrics "linear",
//     "sqeuclidean" and "rbf" (Task Map table; Score Expressions; the SVGD
//     section gives the rbf form exp(-gamma*|x-y|^2)), and "cosine_distances"
//     (Custom Comparisons / Encoded Feature Reuse page, "Prepare Once, Use
//     Several Consumers": 1 - x.y / (|x| |y|), taken as 1 when either vector
//     is zero);
//   * the per-pair score arithmetic applied left to right: scalar multiply
//     and add, add_rows / add_columns, weight_rows / weight_columns and exp
//     (Score Expressions section);
//   * masks that drop pairs from every consumer (Score Expressions: boolean
//     row and column masks; Task Map, Attention row and the note below the
//     Score Expressions example: the pair masks causal, band and
//     same_group). A dropped pair takes no part in the reduction, wherever
//     the mask stands in the op list;
//   * five consumers that reduce each row over j: the kernel product S@V and
//     its row-mass column (Task Map, Nadaraya-Watson row), the displacement
//     sum_j s_ij (y_j - x_i) (SVGD section), the row log-sum-exp with an
//     optional exclusion of the self pair (Task Map, InfoNCE row), the
//     softmax(S)@V product (Intro example, Attention row) and the row top-k
//     with ties broken by lowest index (Task Map, k-NN row; argmin/min row).
//
// It is the plain definition written out: a double loop over pairs, the
// metric in direct form (sum of squared differences, never the norm
// expansion), each reduction two-pass over a per-row buffer of all M scores
// (never online), in higher precision than the inputs: float32 inputs are
// evaluated in double, float64 inputs in x87 80-bit long double. The pages
// state that fused kernels agree with other evaluation orders only within a
// floating tolerance (What to Check, "Precision"), so alongside every result
// the oracle returns a first-order error magnitude `mag` that the tests use
// to scale that tolerance.
//
// Parallelism: OpenMP over rows, nothing else. Build: g++ -O2 -fopenmp
// (no -ffast-math).
//
// Error magnitudes (mu_ij is an upper bound on |s_ij| and on the first-order
// sensitivity of s_ij to unit roundoff in any evaluation order):
//   linear       mu = sum_d |x_d y_d|
//   sqeuclidean  mu = sum_d (|x_d| + |y_d|)^2
//   rbf          mu = k (1 + gamma * sum_d (|x_d| + |y_d|)^2)
//   cosine       mu = 1 + 3 sum_d |x_d y_d| / (|x| |y|)   (1 for a zero vector)
//   MUL c        mu <- |c| mu        (also MUL_ROWS / MUL_COLS with |w_i|, |u_j|)
//   ADD c        mu <- mu + |s_new|  (also ADD_ROWS / ADD_COLS)
//   EXP          mu <- exp(s_old) (1 + mu)
// and per consumer:
//   matmul        mag_c = sum_j (|s_ij| + mu_ij) |V_jc|
//   displacement  mag_d = sum_j (|s_ij| + mu_ij) (|y_jd| + |x_id|)
//   logsumexp     mag   = max_j mu_ij + log(l)   (l = sum_j exp(s_ij - m_i) >= 1)
//   softmax@V     mag_c = sum_j p_ij (1 + mu_ij) |V_jc| + (sum_j p_ij mu_ij)(sum_j p_ij |V_jc|)
//   top-k         mag   = mu of the selected pair
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>
#include <omp.h>

extern "C" {

// Mirrors the Python-side ctypes structure in oracle.py.
typedef struct {
  int dtype;                 // 0: float32 inputs, 1: float64 inputs
  int metric;                // 0: linear, 1: sqeuclidean, 2: rbf, 3: cosine_distances
  double gamma;              // rbf only
  const void *X;             // [N, ldx] row-major, dtype
  int64_t N, ldx;
  const void *Y;             // [M, ldy] row-major, dtype
  int64_t M, ldy;
  int64_t D;
  int n_ops;
  const int *op_kind;        // n_ops entries, see OP_* below
  const double *op_scalar;   // n_ops entries (MUL / ADD)
  const void *const *op_vec; // n_ops entries, host vectors in dtype (ROWS: N, COLS: M)
  // Masks (all optional). A pair (i, j) is kept iff every present mask keeps it.
  const unsigned char *row_mask;  // N entries: row i kept iff nonzero
  const unsigned char *col_mask;  // M entries: column j kept iff nonzero
  int has_upper;                  // kept iff j - i <= upper (causal: upper = 0)
  int64_t upper;
  int has_lower;                  // kept iff i - j <= lower
  int64_t lower;
  const int64_t *group_rows;      // N entries; with group_cols: kept iff
  const int64_t *group_cols;      // group_rows[i] == group_cols[j] (M entries)
} oracle_expr;

}  // extern "C"

namespace {

enum { OP_MUL = 0, OP_ADD = 1, OP_ADD_ROWS = 2, OP_ADD_COLS = 3, OP_MUL_ROWS = 4, OP_MUL_COLS = 5, OP_EXP = 6 };
enum { M_LINEAR = 0, M_SQEUCLIDEAN = 1, M_RBF = 2, M_COSINE = 3 };

inline double rexp(double v) { return std::exp(v); }
inline long double rexp(long double v) { return expl(v); }
inline double rlog(double v) { return std::log(v); }
inline long double rlog(long double v) { return logl(v); }

// One bound expression, inputs of type T, arithmetic in R.
template <class T, class R>
struct Expr {
  const oracle_expr &e;
  const T *X, *Y;
  explicit Expr(const oracle_expr &ex)
      : e(ex), X(static_cast<const T *>(ex.X)), Y(static_cast<const T *>(ex.Y)) {}

  R x(int64_t i, int64_t d) const { return (R)X[i * e.ldx + d]; }
  R y(int64_t j, int64_t d) const { return (R)Y[j * e.ldy + d]; }
  R vec(int k, int64_t idx) const { return (R) static_cast<const T *>(e.op_vec[k])[idx]; }

  // Whether pair (i, j) survives the masks.
  bool keep(int64_t i, int64_t j) const {
    if (e.row_mask && !e.row_mask[i]) return false;
    if (e.col_mask && !e.col_mask[j]) return false;
    if (e.has_upper && j - i > e.upper) return false;
    if (e.has_lower && i - j > e.lower) return false;
    if (e.group_rows && e.group_rows[i] != e.group_cols[j]) return false;
    return true;
  }

  // Score of pair (i, j) with its error magnitude.
  R score(int64_t i, int64_t j, R *mu_out) const {
    R s = 0, mu = 0;
    if (e.metric == M_LINEAR) {
      for (int64_t d = 0; d < e.D; ++d) {
        R p = x(i, d) * y(j, d);
        s += p;
        mu += std::fabs(p);
      }
    } else if (e.metric == M_COSINE) {
      R dot = 0, nx = 0, ny = 0, adot = 0;
      for (int64_t d = 0; d < e.D; ++d) {
        R a = x(i, d), b = y(j, d);
        dot += a * b;
        adot += std::fabs(a * b);
        nx += a * a;
        ny += b * b;
      }
      if (nx > 0 && ny > 0) {
        R den = std::sqrt(nx) * std::sqrt(ny);
        s = 1 - dot / den;
        mu = 1 + 3 * adot / den;
      } else {
        s = 1;
        mu = 1;
      }
    } else {
      R sum_sq = 0, spread = 0;
      for (int64_t d = 0; d < e.D; ++d) {
        R a = x(i, d), b = y(j, d);
        R diff = a - b;
        sum_sq += diff * diff;
        R w = std::fabs(a) + std::fabs(b);
        spread += w * w;
      }
      if (e.metric == M_SQEUCLIDEAN) {
        s = sum_sq;
        mu = spread;
      } else {
        s = rexp(-(R)e.gamma * sum_sq);
        mu = s * (1 + (R)e.gamma * spread);
      }
    }
    for (int k = 0; k < e.n_ops; ++k) {
      switch (e.op_kind[k]) {
        case OP_MUL: s = (R)e.op_scalar[k] * s; mu = std::fabs((R)e.op_scalar[k]) * mu; break;
        case OP_ADD: s = s + (R)e.op_scalar[k]; mu = mu + std::fabs(s); break;
        case OP_ADD_ROWS: s = s + vec(k, i); mu = mu + std::fabs(s); break;
        case OP_ADD_COLS: s = s + vec(k, j); mu = mu + std::fabs(s); break;
        case OP_MUL_ROWS: { R w = vec(k, i); s = w * s; mu = std::fabs(w) * mu; break; }
        case OP_MUL_COLS: { R u = vec(k, j); s = u * s; mu = std::fabs(u) * mu; break; }
        case OP_EXP: { R ex = rexp(s); mu = ex * (1 + mu); s = ex; break; }
        default: break;
      }
    }
    *mu_out = mu;
    return s;
  }
};

template <class T>
using RealOf = typename std::conditional<std::is_same<T, float>::value, double, long double>::type;

int64_t row_at(const int64_t *rows, int64_t r) { return rows ? rows[r] : r; }

// Dense scores (masks are not applied: they act in the consumers).
template <class T>
void do_scores(const oracle_expr &ex, const int64_t *rows, int64_t n_rows, RealOf<T> *out, RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t i = row_at(rows, r);
    for (int64_t j = 0; j < ex.M; ++j) {
      R mu;
      out[r * ex.M + j] = E.score(i, j, &mu);
      mag[r * ex.M + j] = mu;
    }
  }
}

// Kernel product: out[i,c] = sum_j s_ij V[j,c].
template <class T>
void do_matmul(const oracle_expr &ex, const T *V, int64_t C, int64_t ldv, const int64_t *rows, int64_t n_rows,
               RealOf<T> *out, RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t i = row_at(rows, r);
    std::vector<R> acc(C, 0), m(C, 0);
    for (int64_t j = 0; j < ex.M; ++j) {
      if (!E.keep(i, j)) continue;
      R mu;
      R s = E.score(i, j, &mu);
      for (int64_t c = 0; c < C; ++c) {
        R v = (R)V[j * ldv + c];
        acc[c] += s * v;
        m[c] += (std::fabs(s) + mu) * std::fabs(v);
      }
    }
    for (int64_t c = 0; c < C; ++c) {
      out[r * C + c] = acc[c];
      mag[r * C + c] = m[c];
    }
  }
}

// Displacement: out[i,d] = sum_j s_ij (y_jd - x_id), evaluated directly.
template <class T>
void do_displacement(const oracle_expr &ex, const int64_t *rows, int64_t n_rows, RealOf<T> *out, RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
  const int64_t D = ex.D;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t i = row_at(rows, r);
    std::vector<R> acc(D, 0), m(D, 0);
    for (int64_t j = 0; j < ex.M; ++j) {
      if (!E.keep(i, j)) continue;
      R mu;
      R s = E.score(i, j, &mu);
      for (int64_t d = 0; d < D; ++d) {
        R yd = E.y(j, d), xd = E.x(i, d);
        acc[d] += s * (yd - xd);
        m[d] += (std::fabs(s) + mu) * (std::fabs(yd) + std::fabs(xd));
      }
    }
    for (int64_t d = 0; d < D; ++d) {
      out[r * D + d] = acc[d];
      mag[r * D + d] = m[d];
    }
  }
}

// Row log-sum-exp over j, two-pass over the row's buffer of scores.
template <class T>
void do_logsumexp(const oracle_expr &ex, int exclude_self, const int64_t *rows, int64_t n_rows, RealOf<T> *out,
                  RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
#pragma omp parallel
  {
    std::vector<R> s(ex.M), mu(ex.M);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t i = row_at(rows, r);
      int64_t n = 0;
      for (int64_t j = 0; j < ex.M; ++j) {
        if (exclude_self && j == i) continue;
        if (!E.keep(i, j)) continue;
        s[n] = E.score(i, j, &mu[n]);
        ++n;
      }
      if (n == 0) {
        out[r] = -std::numeric_limits<R>::infinity();
        mag[r] = 0;
        continue;
      }
      R m = s[0], mumax = mu[0];
      for (int64_t t = 1; t < n; ++t) {
        m = std::max(m, s[t]);
        mumax = std::max(mumax, mu[t]);
      }
      R l = 0;
      for (int64_t t = 0; t < n; ++t) l += rexp(s[t] - m);
      out[r] = m + rlog(l);
      mag[r] = mumax + rlog(l);
    }
  }
}

// softmax(S)@V over j, two-pass over the row's buffer of scores.
template <class T>
void do_softmax_matmul(const oracle_expr &ex, const T *V, int64_t C, int64_t ldv, const int64_t *rows,
                       int64_t n_rows, RealOf<T> *out, RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
#pragma omp parallel
  {
    std::vector<R> s(ex.M), mu(ex.M), acc(C), av(C), apv(C);
    std::vector<int64_t> jx(ex.M);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t i = row_at(rows, r);
      // The row's kept columns (all of them without masks).
      int64_t n = 0;
      for (int64_t j = 0; j < ex.M; ++j) {
        if (!E.keep(i, j)) continue;
        s[n] = E.score(i, j, &mu[n]);
        jx[n] = j;
        ++n;
      }
      if (n == 0) {
        for (int64_t c = 0; c < C; ++c) out[r * C + c] = mag[r * C + c] = 0;
        continue;
      }
      R m = s[0];
      for (int64_t t = 1; t < n; ++t) m = std::max(m, s[t]);
      R l = 0;
      for (int64_t t = 0; t < n; ++t) l += rexp(s[t] - m);
      std::fill(acc.begin(), acc.end(), (R)0);
      std::fill(av.begin(), av.end(), (R)0);
      std::fill(apv.begin(), apv.end(), (R)0);
      R pmu = 0;
      for (int64_t t = 0; t < n; ++t) {
        const int64_t j = jx[t];
        R p = rexp(s[t] - m) / l;
        pmu += p * mu[t];
        for (int64_t c = 0; c < C; ++c) {
          R v = (R)V[j * ldv + c];
          acc[c] += p * v;
          av[c] += p * (1 + mu[t]) * std::fabs(v);
          apv[c] += p * std::fabs(v);
        }
      }
      for (int64_t c = 0; c < C; ++c) {
        out[r * C + c] = acc[c];
        mag[r * C + c] = av[c] + pmu * apv[c];
      }
    }
  }
}

// Row top-k: the row's kept (s_ij, j) ordered by value (ascending, or
// descending when `largest`), equal values by ascending j; the first
// kk = k + extra are returned, positions past the kept count as NaN / -1.
template <class T>
void do_topk(const oracle_expr &ex, int kk, int largest, const int64_t *rows, int64_t n_rows, RealOf<T> *values,
             int64_t *indices, RealOf<T> *mag) {
  using R = RealOf<T>;
  Expr<T, R> E(ex);
  struct Entry { R v; R mu; int64_t j; };
#pragma omp parallel
  {
    std::vector<Entry> buf(ex.M);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t i = row_at(rows, r);
      int64_t n = 0;
      for (int64_t j = 0; j < ex.M; ++j) {
        if (!E.keep(i, j)) continue;
        buf[n].v = E.score(i, j, &buf[n].mu);
        buf[n].j = j;
        ++n;
      }
      const int64_t keep = std::min<int64_t>(kk, n);
      auto before = [largest](const Entry &a, const Entry &b) {
        if (a.v != b.v) return largest ? (a.v > b.v) : (a.v < b.v);
        return a.j < b.j;
      };
      std::partial_sort(buf.begin(), buf.begin() + keep, buf.begin() + n, before);
      for (int64_t p = 0; p < kk; ++p) {
        if (p < keep) {
          values[r * kk + p] = buf[p].v;
          indices[r * kk + p] = buf[p].j;
          mag[r * kk + p] = buf[p].mu;
        } else {
          values[r * kk + p] = std::numeric_limits<R>::quiet_NaN();
          indices[r * kk + p] = -1;
          mag[r * kk + p] = 0;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ backward
// First-order gradients of each consumer's output, contracted with an
// upstream gradient G, with respect to X, Y, V and every op vector (guide,
// opening section: backward replays the pairs instead of storing them;
// "What to Check", Gradients: selections route gradients through the
// selected pairs only). Written per pair from the chain rule:
//   forward   t_0 = f(x_i, y_j), t_k = op_k(t_{k-1}), s = t_n
//   dS        matmul        G_i . V_j
//             displacement  G_i . (y_j - x_i)
//             logsumexp     g_i exp(s - lse_i)
//             softmax@V     P_ij (G_i . V_j - sum_j' P_ij' G_i . V_j'),  P = exp(s - lse_i)
//             top-k         G_ip at the selected pairs (i, idx_ip), else 0
//   ops       back through the list: MUL c: c d; ADD_ROWS a: grad a_i += d;
//             MUL_ROWS w: grad w_i += d t_{k-1}, d <- w_i d; EXP: d <- d t_k
//             (and the column forms)
//   metric    dX_i += d_0 df/dx_i, dY_j += d_0 df/dy_j with
//             linear df/dx = y; sqeuclidean 2(x - y); rbf -2 gamma f (x - y);
//             cosine -(y/(|x||y|) - (x.y) x/(|x|^3 |y|)) (0 for a zero vector)
//   direct    matmul dV_j += s G_i; softmax dV_j += P_ij G_i;
//             displacement dX_i -= s G_i, dY_j += s G_i
// Masked and excluded pairs contribute nothing. Row-side outputs (dX, row
// op vectors) are returned for a list of rows, column-side outputs (dY,
// dV, column op vectors) for a list of columns; each is computed over all
// pairs it depends on.
//
// `mag` arrays hold each gradient's first-order error magnitude, formed as
// the forward `mag` is: every term contributes its absolute value plus the
// first-order change it takes under unit roundoff in its inputs, with
// mu_k the forward magnitude of t_k and lm_i = max_j mu_ij + log(l_i) that
// of the row's log-sum-exp (the forward log-sum-exp magnitude):
//   dS magnitude  matmul        sum_c |G_ic V_jc|
//                 displacement  sum_d |G_id| (|y_jd| + |x_id|)
//                 logsumexp     |g_i| P (1 + mu + lm_i)
//                 softmax@V     P ((1 + mu + lm_i) |G_i.V_j - D_i| + sum_c |G_ic V_jc| + dm_i),
//                               dm_i = sum_j P_ij ((mu_ij + lm_i) |G_i.V_j| + sum_c |G_ic V_jc|)
//                 top-k         |G| at the selected pairs
//   direct terms  s G: (|s| + mu)|G|;  P G: P (1 + mu + lm_i) |G|
//   ops           MUL c: |c| dm; a weight's gradient d t_k: dm |t_k| + |d| mu_k;
//                 EXP: dm e^t + |d| e^t (1 + mu_k)
//   metric grad   linear |y| (|x|); sqeuclidean 2 (|x| + |y|);
//                 rbf 2 gamma (f + mu_f) (|x| + |y|);
//                 cosine 3 (|y| / (|x||y|) + sum|x y| |x| / (|x|^3 |y|))
//   and each pair adds dm |df| + |d| (that metric-gradient magnitude).
template <class T>
struct Backward {
  using R = RealOf<T>;
  const oracle_expr &ex;
  Expr<T, R> E;
  int consumer;
  const T *G;
  int64_t ldg;
  const T *V;
  int64_t C, ldv;
  int exclude_self;
  const int64_t *idx;
  int k;
  std::vector<R> lse, delta;  // per row, for logsumexp / softmax
  std::vector<R> lm, dmag;    // their first-order magnitudes

  Backward(const oracle_expr &e_, int cons, const T *G_, int64_t ldg_, const T *V_, int64_t C_, int64_t ldv_,
           int excl, const int64_t *idx_, int k_)
      : ex(e_), E(e_), consumer(cons), G(G_), ldg(ldg_), V(V_), C(C_), ldv(ldv_), exclude_self(excl), idx(idx_),
        k(k_) {}

  bool kept(int64_t i, int64_t j) const {
    if (consumer == 2 && exclude_self && i == j) return false;
    return E.keep(i, j);
  }
  R g(int64_t i, int64_t c) const { return (R)G[i * ldg + c]; }
  R v(int64_t j, int64_t c) const { return (R)V[j * ldv + c]; }
  R gv(int64_t i, int64_t j) const {
    R a = 0;
    for (int64_t c = 0; c < C; ++c) a += g(i, c) * v(j, c);
    return a;
  }
  R gv_abs(int64_t i, int64_t j) const {
    R a = 0;
    for (int64_t c = 0; c < C; ++c) a += std::fabs(g(i, c) * v(j, c));
    return a;
  }

  // Per-row log-sum-exp and, for softmax, Delta_i = sum_j P_ij G_i.V_j
  // (two passes over the row, as the forward oracle does).
  void row_stats(int64_t i) {
    R m = -std::numeric_limits<R>::infinity(), mumax = 0;
    for (int64_t j = 0; j < ex.M; ++j) {
      if (!kept(i, j)) continue;
      R mu;
      m = std::max(m, E.score(i, j, &mu));
      mumax = std::max(mumax, mu);
    }
    R l = 0, d = 0;
    if (m != -std::numeric_limits<R>::infinity()) {
      for (int64_t j = 0; j < ex.M; ++j) {
        if (!kept(i, j)) continue;
        R mu;
        R p = rexp(E.score(i, j, &mu) - m);
        l += p;
        if (consumer == 3) d += p * gv(i, j);
      }
    }
    lse[i] = l > 0 ? m + rlog(l) : -std::numeric_limits<R>::infinity();
    delta[i] = l > 0 ? d / l : 0;
    lm[i] = l > 0 ? mumax + rlog(l) : 0;
    // Magnitude of delta_i = sum_j P_ij G_i.V_j (second pass: needs lm_i).
    R dm = 0;
    if (consumer == 3 && l > 0) {
      for (int64_t j = 0; j < ex.M; ++j) {
        if (!kept(i, j)) continue;
        R mu;
        R p = rexp(E.score(i, j, &mu) - lse[i]);
        dm += p * ((mu + lm[i]) * std::fabs(gv(i, j)) + gv_abs(i, j));
      }
    }
    dmag[i] = dm;
  }
  void all_row_stats() {
    if (consumer != 2 && consumer != 3) return;
    lse.assign(ex.N, 0);
    delta.assign(ex.N, 0);
    lm.assign(ex.N, 0);
    dmag.assign(ex.N, 0);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < ex.N; ++i) row_stats(i);
  }

  // Forward values t_0..t_n of pair (i, j) and their magnitudes mu_0..mu_n
  // (propagated as the forward score's magnitude is).
  void forward(int64_t i, int64_t j, R *t, R *mu) const {
    // The metric alone: score() with the ops applied is replayed below.
    oracle_expr bare = ex;
    bare.n_ops = 0;
    Expr<T, R> B(bare);
    t[0] = B.score(i, j, &mu[0]);
    for (int op = 0; op < ex.n_ops; ++op) {
      R x = t[op], m = mu[op];
      switch (ex.op_kind[op]) {
        case OP_MUL: x = (R)ex.op_scalar[op] * x; m = std::fabs((R)ex.op_scalar[op]) * m; break;
        case OP_ADD: x = x + (R)ex.op_scalar[op]; m = m + std::fabs(x); break;
        case OP_ADD_ROWS: x = x + E.vec(op, i); m = m + std::fabs(x); break;
        case OP_ADD_COLS: x = x + E.vec(op, j); m = m + std::fabs(x); break;
        case OP_MUL_ROWS: m = std::fabs(E.vec(op, i)) * m; x = E.vec(op, i) * x; break;
        case OP_MUL_COLS: m = std::fabs(E.vec(op, j)) * m; x = E.vec(op, j) * x; break;
        case OP_EXP: x = rexp(x); m = x * (1 + m); break;
      }
      t[op + 1] = x;
      mu[op + 1] = m;
    }
  }

  // Upstream dS of pair (i, j) and its magnitude, given s and its
  // magnitude mu.
  R dS(int64_t i, int64_t j, R s, R mu, R *scale) const {
    switch (consumer) {
      case 0: *scale = gv_abs(i, j); return gv(i, j);
      case 1: {
        R a = 0, b = 0;
        for (int64_t d = 0; d < ex.D; ++d) {
          R t = g(i, d) * (E.y(j, d) - E.x(i, d));
          a += t;
          b += std::fabs(g(i, d)) * (std::fabs(E.y(j, d)) + std::fabs(E.x(i, d)));
        }
        *scale = b;
        return a;
      }
      case 2: {
        R p = rexp(s - lse[i]);
        *scale = std::fabs((R)G[i * ldg]) * p * (1 + mu + lm[i]);
        return (R)G[i * ldg] * p;
      }
      case 3: {
        R p = rexp(s - lse[i]);
        R a = gv(i, j) - delta[i];
        *scale = p * ((1 + mu + lm[i]) * std::fabs(a) + gv_abs(i, j) + dmag[i]);
        return p * a;
      }
      default: {  // top-k: the selected positions of row i equal to j
        R a = 0;
        for (int p = 0; p < k; ++p)
          if (idx[i * k + p] == j) a += (R)G[i * ldg + p];
        *scale = std::fabs(a);
        return a;
      }
    }
  }

  // df/dx_i (side 0) or df/dy_j (side 1) in out[D] and its magnitude in
  // mag[D], given f = t[0] and its magnitude muf.
  void metric_grad(int64_t i, int64_t j, R f, R muf, int side, R *out, R *mag) const {
    const int64_t D = ex.D;
    if (ex.metric == M_LINEAR) {
      for (int64_t d = 0; d < D; ++d) {
        out[d] = side == 0 ? E.y(j, d) : E.x(i, d);
        mag[d] = std::fabs(out[d]);
      }
    } else if (ex.metric == M_SQEUCLIDEAN || ex.metric == M_RBF) {
      R c = ex.metric == M_SQEUCLIDEAN ? (R)2 : (R)-2 * (R)ex.gamma * f;
      R cm = ex.metric == M_SQEUCLIDEAN ? (R)2 : (R)2 * (R)ex.gamma * (f + muf);
      if (side == 1) c = -c;
      for (int64_t d = 0; d < D; ++d) {
        out[d] = c * (E.x(i, d) - E.y(j, d));
        mag[d] = cm * (std::fabs(E.x(i, d)) + std::fabs(E.y(j, d)));
      }
    } else {
      R dot = 0, nx = 0, ny = 0;
      for (int64_t d = 0; d < D; ++d) {
        dot += E.x(i, d) * E.y(j, d);
        nx += E.x(i, d) * E.x(i, d);
        ny += E.y(j, d) * E.y(j, d);
      }
      if (!(nx > 0 && ny > 0)) {
        for (int64_t d = 0; d < D; ++d) out[d] = mag[d] = 0;
        return;
      }
      R a = std::sqrt(nx), b = std::sqrt(ny), adot = 0;
      for (int64_t d = 0; d < D; ++d) adot += std::fabs(E.x(i, d) * E.y(j, d));
      for (int64_t d = 0; d < D; ++d) {
        if (side == 0) {
          out[d] = -(E.y(j, d) / (a * b) - dot * E.x(i, d) / (a * a * a * b));
          mag[d] = 3 * (std::fabs(E.y(j, d)) / (a * b) + adot * std::fabs(E.x(i, d)) / (a * a * a * b));
        } else {
          out[d] = -(E.x(i, d) / (a * b) - dot * E.y(j, d) / (b * b * b * a));
          mag[d] = 3 * (std::fabs(E.x(i, d)) / (a * b) + adot * std::fabs(E.y(j, d)) / (b * b * b * a));
        }
      }
    }
  }

  // Accumulate pair (i, j) into the side's outputs (row i for side 0,
  // column j for side 1).
  void pair(int64_t i, int64_t j, int side, R *gx, R *gxm, R *gvout, R *gvm, R *gops, R *gopsm) const {
    if (!kept(i, j)) return;
    R t[17], mu[17];
    forward(i, j, t, mu);
    const int n = ex.n_ops;
    R sc;
    R d = dS(i, j, t[n], mu[n], &sc);
    R dm = sc;
    // direct terms
    if (side == 1 && consumer == 0)
      for (int64_t c = 0; c < C; ++c) {
        gvout[c] += t[n] * g(i, c);
        gvm[c] += (std::fabs(t[n]) + mu[n]) * std::fabs(g(i, c));
      }
    if (side == 1 && consumer == 3) {
      R p = rexp(t[n] - lse[i]);
      for (int64_t c = 0; c < C; ++c) {
        gvout[c] += p * g(i, c);
        gvm[c] += p * (1 + mu[n] + lm[i]) * std::fabs(g(i, c));
      }
    }
    if (consumer == 1)
      for (int64_t dd = 0; dd < ex.D; ++dd) {
        R w = t[n] * g(i, dd);
        gx[dd] += side == 0 ? -w : w;
        gxm[dd] += (std::fabs(t[n]) + mu[n]) * std::fabs(g(i, dd));
      }
    // back through the ops
    for (int op = n - 1; op >= 0; --op) {
      const int kind = ex.op_kind[op];
      switch (kind) {
        case OP_MUL: d = (R)ex.op_scalar[op] * d; dm = std::fabs((R)ex.op_scalar[op]) * dm; break;
        case OP_ADD: break;
        case OP_ADD_ROWS:
          if (side == 0) { gops[op] += d; gopsm[op] += dm; }
          break;
        case OP_ADD_COLS:
          if (side == 1) { gops[op] += d; gopsm[op] += dm; }
          break;
        case OP_MUL_ROWS:
          if (side == 0) { gops[op] += d * t[op]; gopsm[op] += dm * std::fabs(t[op]) + std::fabs(d) * mu[op]; }
          d = E.vec(op, i) * d;
          dm = std::fabs(E.vec(op, i)) * dm;
          break;
        case OP_MUL_COLS:
          if (side == 1) { gops[op] += d * t[op]; gopsm[op] += dm * std::fabs(t[op]) + std::fabs(d) * mu[op]; }
          d = E.vec(op, j) * d;
          dm = std::fabs(E.vec(op, j)) * dm;
          break;
        case OP_EXP:
          dm = dm * t[op + 1] + std::fabs(d) * t[op + 1] * (1 + mu[op]);
          d = d * t[op + 1];
          break;
      }
    }
    R mg[64], mgm[64];
    metric_grad(i, j, t[0], mu[0], side, mg, mgm);
    for (int64_t dd = 0; dd < ex.D; ++dd) {
      gx[dd] += d * mg[dd];
      gxm[dd] += dm * std::fabs(mg[dd]) + std::fabs(d) * mgm[dd];
    }
  }
};

template <class T>
void do_backward(const oracle_expr &ex, int consumer, const T *G, int64_t ldg, const T *V, int64_t C, int64_t ldv,
                 int exclude_self, const int64_t *idx, int k, const int64_t *rows, int64_t n_rows,
                 const int64_t *cols, int64_t n_cols, RealOf<T> *dX, RealOf<T> *dXm, RealOf<T> *dY, RealOf<T> *dYm,
                 RealOf<T> *dV, RealOf<T> *dVm, RealOf<T> *dOr, RealOf<T> *dOrm, RealOf<T> *dOc, RealOf<T> *dOcm) {
  using R = RealOf<T>;
  Backward<T> B(ex, consumer, G, ldg, V, C, ldv, exclude_self, idx, k);
  B.all_row_stats();
  const int64_t D = ex.D;
  const int no = ex.n_ops;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t i = rows[r];
    std::vector<R> gx(D, 0), gxm(D, 0), gops(no + 1, 0), gopsm(no + 1, 0);
    for (int64_t j = 0; j < ex.M; ++j) B.pair(i, j, 0, gx.data(), gxm.data(), nullptr, nullptr, gops.data(), gopsm.data());
    for (int64_t d = 0; d < D; ++d) {
      dX[r * D + d] = gx[d];
      dXm[r * D + d] = gxm[d];
    }
    for (int op = 0; op < no; ++op) {
      dOr[op * n_rows + r] = gops[op];
      dOrm[op * n_rows + r] = gopsm[op];
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < n_cols; ++q) {
    const int64_t j = cols[q];
    std::vector<R> gy(D, 0), gym(D, 0), gv(std::max<int64_t>(C, 1), 0), gvm(std::max<int64_t>(C, 1), 0),
        gops(no + 1, 0), gopsm(no + 1, 0);
    for (int64_t i = 0; i < ex.N; ++i)
      B.pair(i, j, 1, gy.data(), gym.data(), gv.data(), gvm.data(), gops.data(), gopsm.data());
    for (int64_t d = 0; d < D; ++d) {
      dY[q * D + d] = gy[d];
      dYm[q * D + d] = gym[d];
    }
    for (int64_t c = 0; c < C; ++c) {
      dV[q * C + c] = gv[c];
      dVm[q * C + c] = gvm[c];
    }
    for (int op = 0; op < no; ++op) {
      dOc[op * n_cols + q] = gops[op];
      dOcm[op * n_cols + q] = gopsm[op];
    }
  }
}

}  // namespace

extern "C" {

// Threads used by every oracle call (0 leaves OpenMP's default).
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
int oracle_max_threads(void) { return omp_get_max_threads(); }

// Size in bytes of the real type results are returned in (8 or sizeof(long double)).
int oracle_real_size(int dtype) { return dtype == 0 ? (int)sizeof(double) : (int)sizeof(long double); }

// For every call below: `rows` lists the global row indices to evaluate
// (NULL means 0..N-1 and then n_rows must equal N); outputs are row-major over
// that list, in double for float32 inputs and long double for float64 inputs.

void oracle_scores(const oracle_expr *e, const int64_t *rows, int64_t n_rows, void *out, void *mag) {
  if (e->dtype == 0) do_scores<float>(*e, rows, n_rows, (double *)out, (double *)mag);
  else do_scores<double>(*e, rows, n_rows, (long double *)out, (long double *)mag);
}

void oracle_matmul(const oracle_expr *e, const void *V, int64_t C, int64_t ldv, const int64_t *rows,
                   int64_t n_rows, void *out, void *mag) {
  if (e->dtype == 0) do_matmul<float>(*e, (const float *)V, C, ldv, rows, n_rows, (double *)out, (double *)mag);
  else do_matmul<double>(*e, (const double *)V, C, ldv, rows, n_rows, (long double *)out, (long double *)mag);
}

void oracle_displacement(const oracle_expr *e, const int64_t *rows, int64_t n_rows, void *out, void *mag) {
  if (e->dtype == 0) do_displacement<float>(*e, rows, n_rows, (double *)out, (double *)mag);
  else do_displacement<double>(*e, rows, n_rows, (long double *)out, (long double *)mag);
}

void oracle_logsumexp(const oracle_expr *e, int exclude_self, const int64_t *rows, int64_t n_rows, void *out,
                      void *mag) {
  if (e->dtype == 0) do_logsumexp<float>(*e, exclude_self, rows, n_rows, (double *)out, (double *)mag);
  else do_logsumexp<double>(*e, exclude_self, rows, n_rows, (long double *)out, (long double *)mag);
}

void oracle_softmax_matmul(const oracle_expr *e, const void *V, int64_t C, int64_t ldv, const int64_t *rows,
                           int64_t n_rows, void *out, void *mag) {
  if (e->dtype == 0)
    do_softmax_matmul<float>(*e, (const float *)V, C, ldv, rows, n_rows, (double *)out, (double *)mag);
  else
    do_softmax_matmul<double>(*e, (const double *)V, C, ldv, rows, n_rows, (long double *)out,
                              (long double *)mag);
}

void oracle_topk(const oracle_expr *e, int kk, int largest, const int64_t *rows, int64_t n_rows, void *values,
                 int64_t *indices, void *mag) {
  if (e->dtype == 0)
    do_topk<float>(*e, kk, largest, rows, n_rows, (double *)values, indices, (double *)mag);
  else
    do_topk<double>(*e, kk, largest, rows, n_rows, (long double *)values, indices, (long double *)mag);
}

// Backward of `consumer` (0 matmul, 1 displacement, 2 logsumexp, 3 softmax
// matmul, 4 top-k) contracted with G: row-side outputs for `rows`
// (dX [n_rows, D], row-op grads [n_ops, n_rows]) and column-side outputs for
// `cols` (dY [n_cols, D], dV [n_cols, C], column-op grads [n_ops, n_cols]);
// each with its absolute-term scale (the *_mag arrays). G is [N, ldg]: C
// columns (matmul, softmax), D (displacement), 1 (logsumexp), k (top-k,
// with the forward's indices idx [N, k]).
void oracle_backward(const oracle_expr *e, int consumer, const void *G, int64_t ldg, const void *V, int64_t C,
                     int64_t ldv, int exclude_self, const int64_t *idx, int k, const int64_t *rows, int64_t n_rows,
                     const int64_t *cols, int64_t n_cols, void *dX, void *dXm, void *dY, void *dYm, void *dV,
                     void *dVm, void *dOr, void *dOrm, void *dOc, void *dOcm) {
  if (e->dtype == 0)
    do_backward<float>(*e, consumer, (const float *)G, ldg, (const float *)V, C, ldv, exclude_self, idx, k, rows,
                       n_rows, cols, n_cols, (double *)dX, (double *)dXm, (double *)dY, (double *)dYm, (double *)dV,
                       (double *)dVm, (double *)dOr, (double *)dOrm, (double *)dOc, (double *)dOcm);
  else
    do_backward<double>(*e, consumer, (const double *)G, ldg, (const double *)V, C, ldv, exclude_self, idx, k, rows,
                        n_rows, cols, n_cols, (long double *)dX, (long double *)dXm, (long double *)dY,
                        (long double *)dYm, (long double *)dV, (long double *)dVm, (long double *)dOr,
                        (long double *)dOrm, (long double *)dOc, (long double *)dOcm);
}

}  // extern "C"
