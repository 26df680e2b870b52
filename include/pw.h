/*
 * pw.h -- C ABI of libpw, lazy pairwise scores reduced on the fly on an
 * AMD Instinct MI355X (gfx950).
 *
 * A pairwise score s_ij = f(x_i, y_j) is bound once (pw_bind) over row-major
 * feature matrices X [N, D] and Y [M, D], then consumed by one of five fused
 * row reductions over j. The [N, M] score matrix is never stored: every call
 * evaluates its pairs tile by tile in bounded device memory, so memory scales
 * with (N + M) * (D + C) plus a caller-provided workspace (torchpairwise
 * guide "Using Torchpairwise in Models", opening section).
 *
 * Conventions shared by every function:
 *  - Return value: PW_OK (0) or a negative pw_status. All validation runs on
 *    the host before any device work; on an error nothing is launched and no
 *    output is written.
 *  - Device pointers (X, Y, op vectors, V, outputs, workspace) are memory of
 *    the current HIP device (e.g. from PyTorch), owned by the caller. A
 *    pw_expr only borrows them: keep them alive and unmodified until the
 *    stream work of every consumer call that uses them has completed.
 *  - Consumers are asynchronous: they enqueue kernels on `stream` (a
 *    hipStream_t; NULL is the null stream) and return. They never allocate
 *    device memory and never synchronise.
 *  - Element type of every floating array is the bound dtype (float or
 *    double); top-k indices are int64_t. Matrices are row-major with the
 *    given leading dimension (elements between consecutive rows).
 *  - A pw_expr is immutable after pw_bind; concurrent consumer calls on one
 *    handle are safe if each gets its own workspace and outputs.
 *  - Results agree with other evaluation orders within floating tolerance,
 *    not bitwise (guide, "What to Check", Precision); for a fixed handle,
 *    consumer and argument set, repeated calls are bitwise identical.
 */
#ifndef PW_H
#define PW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pw_expr pw_expr; /* opaque host-side handle */

typedef enum {
  PW_OK = 0,
  PW_ERR_INVALID = -1,     /* null pointer, bad enum, bad size or stride, k > M, ... */
  PW_ERR_UNSUPPORTED = -2, /* valid request outside the fused range (D not in 1..64, k > 64, > PW_MAX_OPS ops) */
  PW_ERR_WORKSPACE = -3,   /* workspace missing or smaller than pw_workspace_size reports */
  PW_ERR_HIP = -4,         /* a HIP runtime error was reported while enqueueing */
  PW_ERR_SCRATCH = -5      /* pw_topk_noalloc: the call needs more workspace than its static buffer */
} pw_status;

typedef enum { PW_F32 = 0, PW_F64 = 1 } pw_dtype;

/* Built-in metrics (guide, Task Map; rbf form from the SVGD section; cosine
 * from the Custom Comparisons / Encoded Feature Reuse page, "Prepare Once,
 * Use Several Consumers"):
 *   PW_LINEAR       f = sum_d x_d y_d
 *   PW_SQEUCLIDEAN  f = sum_d (x_d - y_d)^2      (squared, no root)
 *   PW_RBF          f = exp(-gamma * sum_d (x_d - y_d)^2), gamma >= 0
 *   PW_COSINE       f = 1 - x.y / (|x| |y|), and 1 when x or y is zero */
typedef enum { PW_LINEAR = 0, PW_SQEUCLIDEAN = 1, PW_RBF = 2, PW_COSINE = 3 } pw_metric;

/* Score arithmetic applied to f left to right, in the order given
 * (guide, "Score Expressions": scalar arithmetic, add_rows, add_columns,
 * weight_rows, weight_columns, exp):
 *   PW_OP_MUL             s <- scalar * s    (division by t is MUL 1/t)
 *   PW_OP_ADD             s <- s + scalar
 *   PW_OP_ADD_ROWS        s <- s + vec[i]    vec: N elements
 *   PW_OP_ADD_COLUMNS     s <- s + vec[j]    vec: M elements
 *   PW_OP_WEIGHT_ROWS     s <- vec[i] * s    vec: N elements
 *   PW_OP_WEIGHT_COLUMNS  s <- vec[j] * s    vec: M elements
 *   PW_OP_EXP             s <- exp(s)
 * `vec` is a contiguous device array of the bound dtype (NULL for MUL, ADD,
 * EXP); `scalar` is rounded to the bound dtype once. */
/* Masks drop pairs (i, j) from every consumer, wherever they stand in the
 * op list (guide, "Score Expressions": boolean row and column masks; Task
 * Map, Attention row, and the note after the Score Expressions example:
 * the pair masks causal, band and same_group). A dropped pair takes no part
 * in the reduction:
 *   PW_OP_MASK_ROWS       keep row i iff vec[i] != 0     vec: N bytes (uint8)
 *   PW_OP_MASK_COLUMNS    keep column j iff vec[j] != 0  vec: M bytes (uint8)
 *   PW_OP_BAND_UPPER      keep iff j - i <= scalar   (causal: scalar = 0)
 *   PW_OP_BAND_LOWER      keep iff i - j <= scalar   (band(lo, hi) is
 *                         BAND_LOWER lo and BAND_UPPER hi)
 *   PW_OP_GROUP_ROWS      row group ids,    vec: N int64_t
 *   PW_OP_GROUP_COLUMNS   column group ids, vec: M int64_t; with GROUP_ROWS
 *                         (both or neither): keep iff g_rows[i] == g_cols[j]
 * Band scalars are integers (|scalar| <= 2^53). At most one mask of each
 * vector kind; several band bounds of one kind keep the tightest. A row whose
 * pairs are all dropped gets the empty-row result of its consumer (zeros,
 * -inf log-sum-exp, zero softmax product, top-k positions NaN / -1). Whole
 * tiles outside a band, or whose row and column group ranges are disjoint,
 * are skipped. */
typedef enum {
  PW_OP_MUL = 0,
  PW_OP_ADD = 1,
  PW_OP_ADD_ROWS = 2,
  PW_OP_ADD_COLUMNS = 3,
  PW_OP_WEIGHT_ROWS = 4,
  PW_OP_WEIGHT_COLUMNS = 5,
  PW_OP_EXP = 6,
  PW_OP_MASK_ROWS = 7,
  PW_OP_MASK_COLUMNS = 8,
  PW_OP_BAND_UPPER = 9,
  PW_OP_BAND_LOWER = 10,
  PW_OP_GROUP_ROWS = 11,
  PW_OP_GROUP_COLUMNS = 12
} pw_op_kind;

#define PW_MAX_OPS 16
#define PW_MAX_D 64
#define PW_MAX_K 64

typedef struct {
  int kind;          /* pw_op_kind */
  double scalar;     /* MUL, ADD, BAND_UPPER, BAND_LOWER */
  const void *vec;   /* ROWS / COLUMNS ops and masks: device vector, borrowed */
} pw_op;

typedef enum {
  PW_C_MATMUL = 0,
  PW_C_DISPLACEMENT = 1,
  PW_C_LOGSUMEXP = 2,
  PW_C_SOFTMAX_MATMUL = 3,
  PW_C_TOPK = 4
} pw_consumer;

/* Bind a lazy score (the `tp.lazy(X, Y, metric, gamma=...)` call of the
 * guide's Task Map, followed by its score arithmetic). Host-only: validates
 * and records pointers, shapes and the op chain; launches nothing and
 * evaluates no pair.
 *   out     receives a new handle (set to NULL on error)
 *   dtype   pw_dtype of X, Y and every op vector
 *   metric  pw_metric; gamma used by PW_RBF only (finite, >= 0)
 *   X       [N, ldx] device matrix, rows are x_i;   N >= 0, ldx >= D
 *   Y       [M, ldy] device matrix, rows are y_j;   M >= 0, ldy >= D
 *           X and Y may be the same pointer (scores of a set with itself)
 *   D       features, 1..PW_MAX_D (PW_ERR_UNSUPPORTED outside that range)
 *   ops     n_ops entries (0..PW_MAX_OPS), copied; op vectors are borrowed.
 *           PW_ERR_UNSUPPORTED when the score arithmetic needs more than 8
 *           fused stages; PW_ERR_INVALID for a second mask of one vector
 *           kind or group ids on one side only
 * X and Y must be aligned to their element size. */
int pw_bind(pw_expr **out, int dtype, int metric, double gamma, const void *X, int64_t N, int64_t ldx,
            const void *Y, int64_t M, int64_t ldy, int64_t D, const pw_op *ops, int n_ops);

/* Bind a score over leading batch elements (torchpairwise "Custom
 * Comparisons / Encoded Feature Reuse" page: one input of batch one against
 * a batch of B; guide, Task Map, MMD row: one feature set per element).
 * Element b scores the rows of X + b*sx against those of Y + b*sy with the
 * same metric and op chain, op t's vector taken at vec + b*op_stride[t];
 * every consumer then runs all B elements in one launch (the tile grid's
 * third dimension). Strides count elements of the dtype; 0 shares one
 * array among all elements (X [1, N, D] against Y [B, M, D] is sx = 0,
 * sy = M*ldy). Masks are shared by every element: op_stride of a mask or a
 * scalar op must be 0. Consumers on a batched handle read V at V + b*sv and
 * write each element's outputs packed one after another: out [B][N][ldo],
 * log-sum-exp and lse [B][N], top-k values and indices [B][N][k] (indices
 * within the element). Backward and CG solves take unbatched handles
 * (PW_ERR_UNSUPPORTED on a batched one).
 *   batch->B   1..65535 (PW_ERR_UNSUPPORTED above); all strides >= 0 */
typedef struct {
  int64_t B;
  int64_t sx, sy;                 /* X, Y */
  int64_t sv;                     /* V of the value consumers */
  int64_t op_stride[PW_MAX_OPS];  /* per op of the list */
} pw_batch;
int pw_bind_batched(pw_expr **out, int dtype, int metric, double gamma, const void *X, int64_t N, int64_t ldx,
                    const void *Y, int64_t M, int64_t ldy, int64_t D, const pw_op *ops, int n_ops,
                    const pw_batch *batch);

/* Free a handle (host memory only). NULL is ignored. */
void pw_release(pw_expr *e);

/* Bytes of device workspace `consumer` needs on this handle (all batch
 * elements of a batched one): C value
 * columns for PW_C_MATMUL / PW_C_SOFTMAX_MATMUL (ignored otherwise) and k
 * for PW_C_TOPK (ignored otherwise). The size depends on N, M, D, C, k and
 * the op chain, never on N*M (the guide's introduction: beyond the inputs and outputs, the
 * streamed path needs only scratch sized by its tiles); it may be 0. */
int pw_workspace_size(const pw_expr *e, int consumer, int64_t C, int k, size_t *bytes);

/* Kernel product (guide, Task Map, "Kernel attention, Nadaraya-Watson" row:
 * `lazy @ V`; with V = [V, ones] the last column is the row mass):
 *   out[i, c] = sum_j s_ij V[j, c]
 *   V    [M, ldv] device matrix, 1 <= C, ldv >= C
 *   out  [N, ldo] device matrix, ldo >= C.  M == 0 writes zeros. */
int pw_matmul(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *ws,
              size_t ws_bytes, void *stream);

/* Displacement (guide, Stein Variational Gradient Descent section: the
 * kernel's displacement, sum_j k_ij (x_j - x_i) for an rbf kernel of a set
 * with itself; for any bound score and Y it is):
 *   out[i, d] = sum_j s_ij (Y[j, d] - X[i, d])
 *   out  [N, ldo] device matrix, ldo >= D.  M == 0 writes zeros. */
int pw_displacement(const pw_expr *e, void *out, int64_t ldo, void *ws, size_t ws_bytes, void *stream);

/* Row log-sum-exp (guide, Task Map, InfoNCE row:
 * `logsumexp(-1, exclude_self=True)`):
 *   out[i] = log sum_{j in J_i} exp(s_ij),  J_i = {0..M-1} minus {i} when
 *   exclude_self (the pair j == i, by index, whatever its value).
 *   out  [N] device vector. An empty J_i gives -inf. */
int pw_logsumexp(const pw_expr *e, int exclude_self, void *out, void *ws, size_t ws_bytes, void *stream);

/* Attention-style product (guide, opening example and Task Map, Attention
 * row: `softmax_matmul(V)`, softmax over the last axis j):
 *   out[i, c] = sum_j softmax_j(s_i.)[j] V[j, c]
 *   V    [M, ldv] device matrix, 1 <= C, ldv >= C
 *   out  [N, ldo] device matrix, ldo >= C.  M == 0 writes zeros. */
int pw_softmax_matmul(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *ws,
                      size_t ws_bytes, void *stream);

/* softmax@V as pw_softmax_matmul, also writing each row's log-sum-exp of the
 * scores, lse[i] = log sum_j exp(s_ij) (-inf for a row with no kept pair),
 * the per-row statistic the backward replays with (guide, opening section:
 * backward by replay; pw_grad_in.lse). lse: N elements of the bound dtype. */
int pw_softmax_matmul_lse(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *lse,
                          void *ws, size_t ws_bytes, void *stream);

/* Row top-k (guide, Task Map, k-NN row `topk(k, largest=False)` with exact
 * tie order, and Chamfer row: min/argmin are k = 1):
 * the k pairs of each row that come first when ordered by s_ij ascending
 * (descending if `largest`), equal values by ascending j; written in that
 * order.
 *   k        0..min(M, PW_MAX_K); k > M is PW_ERR_INVALID, k > PW_MAX_K is
 *            PW_ERR_UNSUPPORTED; k == 0 is a no-op
 *   values   [N, k] device matrix (contiguous) of the bound dtype
 *   indices  [N, k] device matrix (contiguous) of int64_t column indices j
 * NaN scores are unsupported. */
int pw_topk(const pw_expr *e, int k, int largest, void *values, int64_t *indices, void *ws, size_t ws_bytes,
            void *stream);

/* Row top-k as pw_topk, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same plan and kernels, with the workspace taken from a
 * static device buffer of PW_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends. The caller passes inputs
 * and outputs as for pw_topk; the stream must belong to the current device.
 * Calls that need more workspace than the buffer holds (pw_workspace_size
 * of PW_C_TOPK above PW_NOALLOC_SCRATCH_BYTES) return PW_ERR_SCRATCH before
 * any device work. Every call on one GPU shares that GPU's buffer: calls
 * that overlap on one GPU (two streams, two host threads) race; calls in
 * stream order do not. Allocates nothing, ever. */
#define PW_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pw_topk_noalloc(const pw_expr *e, int k, int largest, void *values, int64_t *indices, void *stream);

/* Row mean over the kept pairs (Features page, Native Deployment: the mean
 * reduction over the last dim; guide, Score Expressions: masks decide which
 * pairs a row reduces over):
 *   out[i] = (sum of s_ij over kept j) / (number of kept j),
 * NaN for a row with no kept pair (every row when M == 0). The sums are the
 * kernel product with a column of ones; with masks in the op list, the
 * counts are a second product that scores each kept pair 1 (exact for
 * counts up to 2^24 in float32); a small kernel divides.
 *   out         [N] device vector of the bound dtype ([B][N] on a batched
 *               handle)
 *   inv_counts  optional [N] device vector (NULL to skip): 1 / (number of
 *               kept j), 0 for a row with none; the same for every batch
 *               element. With an appended weight_rows op of this vector, the
 *               kernel product with ones is the mean again, and pw_backward
 *               of that product is the mean's backward.
 * Workspace: pw_mean_workspace_size bytes, caller-owned. */
int pw_mean_workspace_size(const pw_expr *e, size_t *bytes);
int pw_mean(const pw_expr *e, void *out, void *inv_counts, void *ws, size_t ws_bytes, void *stream);

/* Squared maximum mean discrepancy between point clouds (guide, Task Map,
 * MMD row: mmd_statistics of [B, n, D] and [B, m, D] clouds, one feature set
 * per cloud, unbiased by default), under the kernel k given by `metric` and
 * `gamma` (any built-in metric; all are symmetric):
 *   unbiased: sum_{i != i'} k(x_i, x_i') / (n (n-1))
 *             + sum_{j != j'} k(y_j, y_j') / (m (m-1)) - 2 sum_{i,j} k(x_i, y_j) / (n m)
 *   biased:   the within-cloud sums over all pairs, over n^2 and m^2.
 * The three sums are kernel products with a column of ones; a within-cloud
 * sum of the unbiased statistic takes the strict upper triangle (a band
 * mask: half the pairs) and doubles it. One kernel per batch element adds
 * the row sums in double and forms the statistic.
 *   X     element b's cloud at X + b*sx ([n, ldx] row-major, dtype); sx = 0
 *         shares one cloud across the batch; likewise Y, m, ldy, sy
 *   B     1..65535 batch elements; n, m >= 2 (unbiased) or >= 1 (biased);
 *         D 1..PW_MAX_D
 *   out   [B] device vector of the dtype
 * Workspace: pw_mmd2_workspace_size bytes, caller-owned. Errors as pw_bind
 * (PW_ERR_INVALID / PW_ERR_UNSUPPORTED) before any device work. */
int pw_mmd2_workspace_size(int dtype, int metric, double gamma, int64_t n, int64_t m, int64_t D, int64_t B,
                           size_t *bytes);
int pw_mmd2(int dtype, int metric, double gamma, const void *X, int64_t n, int64_t ldx, int64_t sx, const void *Y,
            int64_t m, int64_t ldy, int64_t sy, int64_t D, int64_t B, int unbiased, void *out, void *ws,
            size_t ws_bytes, void *stream);

/* Gradients of sum_b G[b] * MMD2_b (the statistics of pw_mmd2 with the same
 * arguments) with respect to both clouds (Task Map: every row has
 * first-order gradients; guide, opening section: a backward replays the
 * pairs). Each of the three sums is a kernel product with ones, so its
 * gradient is pw_backward of that product (row and column sides) with a
 * column of ones as upstream gradient; a kernel then adds the sides with
 * the statistic's coefficients, scaled by G[b]. Batch elements run one after
 * another (the backward takes unbatched products).
 *   G     [B] device vector (dtype): upstream gradient of each statistic
 *   dX    [B][n][lddx] (sx > 0), or [n][lddx] (sx == 0: the gradient of the
 *         shared cloud, summed over the batch), or NULL if not wanted;
 *         lddx >= D; dY, lddy likewise for Y. Outputs are overwritten.
 * Workspace: pw_mmd2_backward_workspace_size bytes. Errors as pw_mmd2. */
int pw_mmd2_backward_workspace_size(int dtype, int metric, double gamma, int64_t n, int64_t m, int64_t D,
                                    size_t *bytes);
int pw_mmd2_backward(int dtype, int metric, double gamma, const void *X, int64_t n, int64_t ldx, int64_t sx,
                     const void *Y, int64_t m, int64_t ldy, int64_t sy, int64_t D, int64_t B, int unbiased,
                     const void *G, void *dX, int64_t lddx, void *dY, int64_t lddy, void *ws, size_t ws_bytes,
                     void *stream);

/* ------------------------------------------------------------------------
 * Backward by replay (guide, opening section: the consumer's backward
 * re-evaluates the pairs instead of keeping the [N, M] matrix; "What to
 * Check", Gradients: selections route gradients through the selected pairs
 * only). Given the upstream gradient G of a consumer's output, returns the
 * gradients of sum(output * G) with respect to X, Y, V and the vector of
 * every op, each pair's contribution formed from the chain rule on the fly.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *G;           /* [N, ldg] upstream gradient: C columns (matmul, softmax),
                              D (displacement), 1 (logsumexp), k (top-k) */
  int64_t ldg;
  const void *V;           /* matmul, softmax: the forward call's V [M, ldv], C columns */
  int64_t C, ldv;
  const void *out;         /* softmax: the forward output [N, ldo] (required);
                              logsumexp: the forward output [N] (NULL: recomputed) */
  int64_t ldo;
  const int64_t *indices;  /* top-k: the forward call's indices [N, k] (-1 entries skipped) */
  int k;
  int exclude_self;        /* logsumexp: as in the forward call */
  const void *lse;         /* softmax: the forward's row log-sum-exp [N] from
                              pw_softmax_matmul_lse, or NULL (recomputed) */
} pw_grad_in;

typedef struct {
  void *dX;                /* [N, lddx] gradient of X, or NULL */
  int64_t lddx;
  void *dY;                /* [M, lddy] gradient of Y, or NULL */
  int64_t lddy;
  void *dV;                /* [M, lddv] gradient of V (matmul, softmax), or NULL */
  int64_t lddv;
  void *dops[PW_MAX_OPS];  /* entry t: gradient of op t's vector (N or M elements) for
                              ADD/WEIGHT_ROWS/COLUMNS ops, else ignored; NULL: not wanted */
} pw_grad_out;

/* Describe the kernels pw_backward would run for `consumer` and C value
 * columns when no op-vector gradient is asked (want_ops = 0) or some is
 * (want_ops = 1): the matrix-core backward or the vector backward engine. */
int pw_backward_plan_describe(const pw_expr *e, int consumer, int64_t C, int want_ops, char *buf, size_t len);

/* Workspace bytes of pw_backward for `consumer`, C value columns, k. */
int pw_backward_workspace_size(const pw_expr *e, int consumer, int64_t C, int k, size_t *bytes);

/* Gradients of sum(consumer output * G): every requested output is
 * overwritten. Masks and the excluded self pair contribute nothing. For
 * X aliasing Y (one set with itself) dX and dY are the two sides' parts;
 * the set's gradient is their sum. Supported: every metric, op and mask;
 * D <= 64; C <= 64 (PW_ERR_UNSUPPORTED above). Top-k column gradients
 * (dY, column ops) are summed with atomics: not bitwise repeatable. */
int pw_backward(const pw_expr *e, int consumer, const pw_grad_in *in, const pw_grad_out *out, void *ws,
                size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Conjugate-gradient solve (guide, Task Map, "Kernel ridge, GP mean" row:
 * solve(K + a * eye_like(K), Y, method="cg"); "What to Check", Solvers:
 * results carry converged and status, to be checked before the solution is
 * used). The product with K in every iteration is pw_matmul's fused tile
 * path; the vector steps are small reduction kernels of this library.
 * ---------------------------------------------------------------------- */
typedef enum {
  PW_SOLVE_CONVERGED = 0, /* every column reached |r_c| <= rtol |b_c| */
  PW_SOLVE_MAX_ITER = 1,  /* max_iter iterations without reaching it */
  PW_SOLVE_BREAKDOWN = 2  /* p.(S + shift I)p <= 0 in some column: not positive definite */
} pw_solve_status;

typedef struct {
  int converged;           /* 1 iff status == PW_SOLVE_CONVERGED */
  int status;              /* pw_solve_status */
  int iterations;          /* iterations run (the last check's count) */
  double max_rel_residual; /* max over columns of |r_c| / |b_c| from the CG recurrence */
} pw_solve_info;

/* Bytes of device workspace pw_cg_solve needs for C right-hand sides. */
int pw_cg_workspace_size(const pw_expr *e, int64_t C, size_t *bytes);

/* Solve (S + shift I) A = B by conjugate gradients from A = 0, for a square
 * bound score S (N == M) that is symmetric positive semi-definite (e.g. an
 * rbf kernel of a set with itself), column by column:
 *   shift       > 0 (finite)
 *   B           [N, ldb] device matrix, C right-hand sides, 1 <= C, ldb >= C
 *   A           [N, lda] device matrix, the solution (overwritten)
 *   max_iter    >= 1; rtol >= 0 per column: stop when |r_c| <= rtol |b_c|
 *   check_every >= 1: iterations between the host's convergence checks
 *   info        host struct, filled on PW_OK
 * Columns that converge are frozen; a zero column of B gives a zero column
 * of A. Unlike the consumers, this call synchronises `stream` at every
 * convergence check (a small device-to-host copy) and on return. The
 * workspace must not be used by other work until the call returns. */
int pw_cg_solve(const pw_expr *e, double shift, const void *B, int64_t C, int64_t ldb, void *A, int64_t lda,
                int max_iter, double rtol, int check_every, void *ws, size_t ws_bytes, void *stream,
                pw_solve_info *info);

/* Describe the launch plan `consumer` would use (kernel family, tile sizes,
 * column splits) into buf as a NUL-terminated string. For logs and tuning. */
int pw_plan_describe(const pw_expr *e, int consumer, int64_t C, int k, char *buf, size_t len);

/* Profiling hook for benchmarks: after this call, every consumer call made
 * by the calling thread records the hipEvent_t `start` on its stream just
 * before its main tile-kernel launch and `stop` just after it (for value
 * widths above one launch's chunk, around all of the call's tile launches).
 * The events are created and owned by the caller; NULL, NULL disables the
 * hook. Thread-local: other threads are unaffected. Never fails.
 * pw_backward records the pair around all of its tile launches (both
 * sides, with the small merges between them). */
int pw_set_tile_events(void *start, void *stop);

/* Static text for a pw_status code. */
const char *pw_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* PW_H */
