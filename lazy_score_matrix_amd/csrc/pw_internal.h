// Internal structures shared by the libpw host code and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

// ---------------------------------------------------------------------------
// Canonical score epilogue.
//
// The score arithmetic of the guide's "Score Expressions" section (scalar
// multiply/add, add_rows, add_columns, weight_rows, weight_columns, exp) is
// compiled at bind time into at most kMaxStages stages, applied in order:
//   affine:  s <- s * (r_i * q_j) + (p_i + o_j)
//   exp:     s <- exp(s)
// Consecutive ops fold into one affine stage while the result stays of this
// separable form; an op that would break it (a column weight after a row
// offset, a row weight after a column offset) starts a new stage. r_i, p_i
// are uniform scalars or per-row vectors, q_j, o_j per-column vectors; the
// vectors are evaluated once per consumer call into the workspace by a
// pre-pass (vector programs below), in double, then rounded to the dtype.
// ---------------------------------------------------------------------------
constexpr int kMaxStages = 8;
enum StageKind : int { ST_AFFINE = 0, ST_EXP = 1 };

struct Stage {
  int kind;         // StageKind
  int row_vec;      // r_i, p_i read from r_vec / p_vec (else r_scalar / p_scalar)
  int col_vec;      // q_j, o_j read from q_vec / o_vec (else 1 and 0)
  double r_scalar;
  double p_scalar;
  const void *r_vec, *p_vec;  // N elements of the dtype, in the workspace
  const void *q_vec, *o_vec;  // M elements of the dtype, in the workspace
};

struct Epi {
  int n_stages;
  int any_col;  // some stage has column vectors
  Stage st[kMaxStages];
};

// Vector program: out[e] = evaluation of `ins` at element e, in double.
enum VecOp : int { VO_SET = 0, VO_MULC = 1, VO_ADDC = 2, VO_MULV = 3, VO_ADDV = 4 };
constexpr int kMaxVecInstr = 12;
struct VecInstr {
  int op;
  double c;
  const void *v;    // dtype vector for VO_MULV / VO_ADDV
  int64_t bstride;  // bytes between the vectors of consecutive batch elements (0: shared)
};
struct VecProg {
  int n;
  int64_t len;
  void *out;            // dtype vector of `len` elements
  int64_t out_bstride;  // bytes between consecutive batch elements' outputs
  VecInstr ins[kMaxVecInstr];
};
constexpr int kProgsPerLaunch = 6;
struct VecProgBatch {
  int n_progs;
  VecProg p[kProgsPerLaunch];
};

enum Consumer : int { C_MATMUL = 0, C_DISPLACEMENT = 1, C_LOGSUMEXP = 2, C_SOFTMAX = 3, C_TOPK = 4 };
enum Metric : int { M_LINEAR = 0, M_SQEUCLIDEAN = 1, M_RBF = 2, M_COSINE = 3 };

// ---------------------------------------------------------------------------
// Arguments of one tile-engine launch.
//
// The grid covers (row block) x (column split). Each workgroup reduces its
// rows over one contiguous column range; with n_split > 1 it writes a
// partial (per-row sums, (max, sum[, acc]) pairs or sorted top-k keys) to
// the workspace and a merge kernel combines the splits in a fixed order.
// ---------------------------------------------------------------------------
// Masks: pairs dropped from every consumer. Tiles are classified per row
// block and key tile: skipped, checked pair by pair, or kept whole.
struct MaskArgs {
  const uint8_t *row;       // N bytes: row i kept iff nonzero (null: all)
  const uint8_t *col;       // M bytes: column j kept iff nonzero (null: all)
  int band;                 // lo/hi bounds present
  int64_t lo, hi;           // kept iff lo <= j - i <= hi
  const int64_t *grow;      // row group ids (null: no group mask)
  const int64_t *gcol;      // column group ids: kept iff grow[i] == gcol[j]
  const int64_t *grow_rng;  // [n_rb][2] min and max row group per row block
  const int64_t *gcol_rng;  // [ceil(M / bn)][2] min and max per key tile
  const int64_t *span;      // [n_rb][2] first and end column of the tiles a row
                            // block keeps under the pair masks (null: no span)
  int any;                  // any mask present
};
constexpr int64_t kBandNone = (int64_t)1 << 62;

// Batched launches: the grid's z index is the batch element, and each array
// below is offset by z times its stride in bytes (0: one array serves every
// element; an absent array, a null pointer, always has stride 0). Masks and
// their tables are shared by every element.
struct BatchArgs {
  int64_t n;  // batch elements (1: an unbatched call)
  int64_t x, y, v, out, idx, lse, part, ny, epi;
};
constexpr int64_t kMaxBatch = 65535;  // the grid's z extent

struct TileArgs {
  const void *X;
  int64_t ldx;
  const void *Y;
  int64_t ldy;
  int64_t N, M;
  int D;
  double gamma;
  const void *V;  // value matrix (matmul / softmax), already offset to the column chunk
  int64_t ldv;
  int C;          // value columns in this launch
  void *out;      // final output (n_split == 1), already offset to the column chunk
  int64_t ldo;
  void *lse_out;  // softmax: optional row log-sum-exp [N] of the scores (kept for the backward)
  int64_t *idx;   // top-k indices
  int k;
  int largest;
  int exclude_self;
  int n_rb;              // row blocks
  int rb_pairs;          // MFMA masked launches: workgroups per split that each take
                         // row blocks r and n_rb - 1 - r (0: one row block each)
  const int *rb_order;   // with rb_pairs: row blocks by kept tiles, heaviest first, so
                         // pair slot r takes rb_order[r] and rb_order[n_rb - 1 - r]
                         // (null: by index)
  int n_split;           // column splits
  int64_t split_cols;    // columns per split (multiple of the tile width)
  void *partial;         // workspace partials when n_split > 1
  const void *nx;        // unused (row norms are formed in-kernel)
  const void *ny;        // column norms |y_j|^2 (distances) or 1/|y_j| (cosine, 0 for y_j = 0)
  double exp2_c[4];      // (ln2/256)^k / k!, k = 1..4, for the table-driven double exp2
  Epi epi;
  MaskArgs mask;
  BatchArgs bat;
};

// Top-k partial key layouts in the workspace.
//   float:  one uint64 per entry: orderable(value) << 32 | j
//   double: two uint64 per entry: orderable(value), j
template <class T>
struct TopkKeyBytes;
template <>
struct TopkKeyBytes<float> { static constexpr int value = 8; };
template <>
struct TopkKeyBytes<double> { static constexpr int value = 16; };

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files). All return hipError_t of the launch.
// ---------------------------------------------------------------------------
// Generic VALU tile engine: any D <= 64, any metric, consumer and op chain.
//   dtile: feature tile 3 / 4 / 16 / 64 (D zero-padded up to it)
//   vtile: value tile 4 / 16 / 64 (matmul, softmax), top-k list 16 / 64, else 0
struct ValuConfig {
  int dtile;
  int vtile;
  int rows = 1;  // rows per thread (kProdRows: the blocked float kernel product; 2: the
                 // blocked float row minimum and log-sum-exp)
};
template <class T, int METRIC>
hipError_t valu_launch_metric(int consumer, const ValuConfig &cfg, const TileArgs &a, hipStream_t s);
constexpr int kValuBM = 256;  // rows per workgroup (one per thread)
constexpr int kValuBN = 64;   // columns per staged tile
// The plain float kernel product of narrow points: rows per thread, and
// columns per staged tile (one per thread).
constexpr int kProdRows = 4;
constexpr int kProdBN = kValuBM;
// Workgroups per compute unit the planner aims the product at: many short
// workgroups (about 16 per CU, four resident at a time) let the dispatcher
// even out the CUs' finishing times (measured 0.80 ms against 0.89 ms with
// four per CU at 65536 x 65536).
constexpr int kProdWGsPerCU = 16;

// MFMA tile engine: D >= 16, op chains of at most one row-affine stage.
//   dp: feature tile 16 / 32 / 64; cp: value tile (float 32 / 64, double
//   16 / 32 / 64); kl: top-k list 16 / 64.
struct MfmaConfig {
  int dp;
  int cp;
  int kl;
};
// Wide variants (64-slot top-k lists; double with a feature or value tile
// above 16) need the whole 512-register budget: one 4-wave workgroup per CU,
// one wave per SIMD. The others run two 4-wave workgroups per CU (two waves
// per SIMD, 256 registers each). Measured on gfx950, sharing each staged
// tile among 8 waves instead did not pay.
constexpr bool mfma_wide(int dtype, int dp, int cp, int kl) { return kl > 16 || (dtype == 1 && (dp > 16 || cp > 16)); }
constexpr int mfma_waves(int, int, int, int) { return 4; }
// Workgroups per CU (the launch bound): wide register states run one, the
// rest two (three measured no faster for the single-column product).
constexpr int mfma_wgs_per_cu(int dtype, int consumer, int dp, int cp, int kl) {
  return (void)consumer, mfma_wide(dtype, dp, cp, kl) ? 1 : 2;
}
// Query rows per workgroup: waves x QB blocks x (32 float / 16 double)
// queries; double uses QB = 2 except for top-k.
constexpr int mfma_bm(int dtype, int consumer, int dp, int cp, int kl) {
  return mfma_waves(dtype, dp, cp, kl) * ((dtype == 1 && consumer != C_TOPK) ? 2 : 1) * (dtype == 0 ? 32 : 16);
}
// Keys per staged tile: float 128 (4 sub-blocks of 32) except for the value
// consumers with a V tile (cp > 1), whose prefetched tile needs the
// registers, and top-k with more than 32 features, whose candidate queue
// needs the LDS (64); double 64.
constexpr int mfma_bn(int dtype, int consumer, int cp, int dp) {
  return (dtype == 0 && ((consumer != C_MATMUL && consumer != C_SOFTMAX) || cp == 1) &&
          !(consumer == C_TOPK && dp > 32))
             ? 128
             : 64;
}
// Lane groups per query in the MFMA layouts (float 2, double 4); each keeps
// its own top-k list, written as a separate partial.
constexpr int mfma_groups(int dtype) { return dtype == 0 ? 2 : 4; }
template <class T, int METRIC>
hipError_t mfma_launch_metric(int consumer, const MfmaConfig &cfg, const TileArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// Backward by replay (grad_engine.h). The raw arithmetic ops, in order (the
// masks are in MaskArgs); `where` 0 scalar / none, 1 row vector, 2 column.
// ---------------------------------------------------------------------------
constexpr int kGradOps = 16;
struct GradOp {
  int kind;       // PW_OP_* arithmetic kind
  int where;
  double scalar;
  const void *vec;
};
struct GradArgs {
  const void *X, *Y;
  int64_t ldx, ldy, N, M;
  int D;
  double gamma;
  int n_ops;
  GradOp ops[kGradOps];
  int fast;            // ops folded into `stage` (one affine stage), no op grads
  Stage stage;
  const void *G;       // upstream gradient [N, ldg]
  int64_t ldg;
  const void *V;       // forward V [M, ldv] (matmul, softmax)
  int64_t ldv;
  int C;
  const void *lse;     // [N] row log-sum-exp (logsumexp, softmax)
  const void *delta;   // [N] sum_c G_ic O_ic (softmax)
  const void *inv_x;   // [N] 1/|x_i| (cosine)
  const void *inv_y;   // [M] 1/|y_j| (cosine)
  int exclude_self;
  MaskArgs mask;
  const int64_t *idx;  // top-k indices [N, k]
  int k;
  // Partial outputs [n_split][own rows][W]: gradient of the own point (D),
  // then dV (C, column side of value consumers), then one slot per op.
  int n_rb, n_split;
  int64_t split;
  void *partial;
  int W;
  // Top-k writes its outputs directly (row side plain, column side atomic).
  void *dX, *dY;
  int64_t lddx, lddy;
  void *dop[kGradOps];
};
struct GradOut {
  void *own;  // dX (side 0) or dY (side 1)
  int64_t ld_own;
  void *dV;
  int64_t lddv;
  void *dop[kGradOps];  // only the ops on this side are written
};
// Matrix-core backward of dot-product scores s_ij = r_i (x_i . y_j) + p_i
// for softmax@V and logsumexp, float32 (mfma_grad.hip).
struct MfmaGradArgs {
  const float *X, *Y, *V, *G;
  int64_t ldx, ldy, ldv, ldg;
  int64_t N, M;
  int D, C;
  const float *lse;    // [N] row log-sum-exp
  const float *delta;  // [N] G_i . O_i (softmax)
  int row_vec;         // r_i, p_i from r_vec / p_vec, else r_s, p_s
  float r_s, p_s;
  const float *r_vec, *p_vec;
  int exclude_self;
  MaskArgs mask;       // band and row / column masks (no groups on this path)
  int n_rb, n_split;
  int rb_pairs;        // with a band: workgroups per split, each taking own blocks r, n_rb - 1 - r
  int64_t split;
  float *partial;      // [n_split][own rows][W]: own gradient (D), then dV (C, side 1)
  int W;
};
hipError_t mfma_grad_launch(int consumer, int side, int dp, int cp, const MfmaGradArgs &a, hipStream_t s);
int mfma_grad_rows();  // rows per workgroup of the matrix-core backward
hipError_t grad_launch(int dtype, int metric, int consumer, int side, int dt, int ct, const GradArgs &a,
                       hipStream_t s);
hipError_t grad_topk_launch(int dtype, int metric, int dt, const GradArgs &a, hipStream_t s);
hipError_t launch_grad_merge(int dtype, const GradArgs &a, int side, int64_t n_own, int C1, const GradOut &o,
                             hipStream_t s);
hipError_t launch_grad_delta(int dtype, const void *G, int64_t ldg, const void *O, int64_t ldo, int64_t N, int C,
                             void *delta, hipStream_t s);

// Conjugate-gradient vector steps (cg_kernels.hip). Iterates are [N, C]
// row-major with ld C; column partial sums are doubles [cg_blocks(N)][C].
struct CgState {
  double *rr, *bb, *alpha, *beta;  // per column: |r|^2, |b|^2, step sizes
  int *flag;                       // per column: 1 running, 0 converged, 2 breakdown
};
constexpr int kCgRows = 1024;  // rows per reduction block
int cg_blocks(int64_t N);
hipError_t launch_cg_init(int dtype, const void *B, int64_t ldb, void *A, int64_t lda, void *R, void *P, int64_t N,
                          int C, double *part, hipStream_t s);
hipError_t launch_cg_pq(int dtype, const void *P, void *Q, int64_t N, int C, double shift, double *part,
                        hipStream_t s);
hipError_t launch_cg_update(int dtype, const void *P, const void *Q, void *A, int64_t lda, void *R, int64_t N, int C,
                            CgState st, double *part, hipStream_t s);
hipError_t launch_cg_direction(int dtype, const void *R, void *P, int64_t N, int C, CgState st, hipStream_t s);
// phase 0: after init, 1: step sizes alpha, 2: betas and convergence.
hipError_t launch_cg_scalars(int phase, const double *part, int nblk, int C, CgState st, double tol2,
                             hipStream_t s);

// Auxiliary kernels.
hipError_t launch_vec_progs(int dtype, const VecProgBatch &b, int64_t n_batch, hipStream_t s);
// Per block of `block` entries of g[0..n): min and max, written as pairs.
hipError_t launch_group_ranges(const int64_t *g, int64_t n, int block, int64_t *out, hipStream_t s);
// Per row block of bm rows: the column span [first, end) of the key tiles of
// bn columns that the pair masks do not skip ([0, 0) when none).
hipError_t launch_tile_spans(const MaskArgs &m, int64_t N, int64_t M, int bm, int bn, int n_rb, int64_t *out,
                             hipStream_t s);
// Row blocks ordered by the key tiles a paired launch deals them (their band
// and span reach), heaviest first, ties by index; n_rb <= kMaxOrderedBlocks.
constexpr int kMaxOrderedBlocks = 4096;
hipError_t launch_pair_order(const MaskArgs &m, int64_t N, int64_t M, int bm, int bn, int n_rb, int *order,
                             hipStream_t s);
hipError_t launch_fill(int dtype, void *out, int64_t rows, int64_t cols, int64_t ld, double value, hipStream_t s);
// out[b][i] /= kept count of row i (cnt[i], or M when cnt is null); NaN for a
// row with none; inv[i] = 1 / count (0 for none) when inv is not null.
hipError_t launch_mean_finish(int dtype, void *out, int64_t N, int64_t B, const void *cnt, int64_t M, void *inv,
                              hipStream_t s);
// Per batch element b: the squared MMD from the kernel products' row sums
// rxx [B][n], ryy [B][m], rxy [B][n]: cx * sum rxx + cy * sum ryy - cxy * sum
// rxy, the sums in double in a fixed order; out [B].
hipError_t launch_mmd_finish(int dtype, const void *rxx, const void *ryy, const void *rxy, int64_t n, int64_t m,
                             int64_t B, double cx, double cy, double cxy, void *out, hipStream_t s);
// out[i][d] (= or +=) G[b] * (c1 * (a + a2)[i][d] - c2 * c[i][d]) over a [rows][D]
// gradient block; a, a2, c dense [rows][D], out [rows][ldo].
hipError_t launch_mmd_grad_combine(int dtype, const void *a, const void *a2, const void *c, int64_t rows, int64_t D,
                                   const void *G, int64_t b, double c1, double c2, void *out, int64_t ldo,
                                   bool accumulate, hipStream_t s);
// Row norms |x_i|^2, or with `inverse` 1/|x_i| (0 for a zero row).
// With n_batch > 1, element b reads X + b * x_bstride and writes out +
// b * out_bstride (bytes).
hipError_t launch_row_norms(int dtype, const void *X, int64_t n, int64_t ld, int D, void *out, hipStream_t s,
                            bool inverse = false, int64_t n_batch = 1, int64_t x_bstride = 0,
                            int64_t out_bstride = 0);
hipError_t launch_merge(int dtype, int consumer, const TileArgs &a, hipStream_t s);

}  // namespace pw
