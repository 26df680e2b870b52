// libpw C ABI: validation, op-chain compilation, launch planning, workspace
// layout and dispatch. Declarations and semantics: include/pw.h.
#include "../../include/pw.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pw_internal.h"

using namespace pw;

namespace {

// ---------------------------------------------------------------------------
// Op-chain compilation into canonical stages (see pw_internal.h).
// ---------------------------------------------------------------------------
struct Prog {
  std::vector<VecInstr> ins;
  bool vec = false;   // depends on a vector
  double cval = 0.0;  // value when !vec
  void set(double c) {
    ins.assign(1, VecInstr{VO_SET, c, nullptr});
    vec = false;
    cval = c;
  }
  void mulc(double c) {
    ins.push_back(VecInstr{VO_MULC, c, nullptr});
    if (!vec) cval *= c;
  }
  void addc(double c) {
    ins.push_back(VecInstr{VO_ADDC, c, nullptr});
    if (!vec) cval += c;
  }
  // bs: bytes between the vectors of consecutive batch elements (0: shared).
  void mulv(const void *v, int64_t bs) {
    ins.push_back(VecInstr{VO_MULV, 0.0, v, bs});
    vec = true;
  }
  void addv(const void *v, int64_t bs) {
    ins.push_back(VecInstr{VO_ADDV, 0.0, v, bs});
    vec = true;
  }
  bool is_const(double c) const { return !vec && cval == c; }
};

struct HostStage {
  int kind = ST_AFFINE;
  bool row_vec = false, col_vec = false;
  double r_scalar = 1.0, p_scalar = 0.0;
  Prog r, p, q, o;
};

struct StageBuilder {
  std::vector<HostStage> out;
  Prog ar, br, ac, bc;
  StageBuilder() { start(); }
  void start() {
    ar.set(1.0);
    br.set(0.0);
    ac.set(1.0);
    bc.set(0.0);
  }
  void close() {
    const bool row_vec = ar.vec || br.vec, col_vec = ac.vec || bc.vec;
    if (!row_vec && !col_vec && ar.cval == 1.0 && br.cval == 0.0) {
      start();
      return;  // identity
    }
    HostStage s;
    s.kind = ST_AFFINE;
    s.row_vec = row_vec;
    s.col_vec = col_vec;
    s.r_scalar = ar.cval;
    s.p_scalar = br.cval;
    s.r = ar;
    s.p = br;
    s.q = ac;
    s.o = bc;
    out.push_back(s);
    start();
  }
  void op(const pw_op &o, int64_t bs) {
    switch (o.kind) {
      case PW_OP_EXP: {
        close();
        HostStage s;
        s.kind = ST_EXP;
        out.push_back(s);
        break;
      }
      case PW_OP_MUL:
        ar.mulc(o.scalar);
        br.mulc(o.scalar);
        bc.mulc(o.scalar);
        break;
      case PW_OP_ADD: br.addc(o.scalar); break;
      case PW_OP_ADD_ROWS: br.addv(o.vec, bs); break;
      case PW_OP_ADD_COLUMNS: bc.addv(o.vec, bs); break;
      case PW_OP_WEIGHT_ROWS:
        if (bc.vec) close();  // w_i * o_j is not separable: new stage
        ar.mulv(o.vec, bs);
        br.mulv(o.vec, bs);
        break;
      case PW_OP_WEIGHT_COLUMNS:
        if (br.vec) close();  // u_j * p_i is not separable: new stage
        if (!br.is_const(0.0)) {  // a scalar offset moves to the column side
          bc.addc(br.cval);
          br.set(0.0);
        }
        ac.mulv(o.vec, bs);
        bc.mulv(o.vec, bs);
        break;
    }
  }
};

}  // namespace

struct pw_expr {
  int dtype, metric;
  double gamma;
  const void *X;
  int64_t N, ldx;
  const void *Y;
  int64_t M, ldy;
  int64_t D;
  std::vector<pw_op> ops;
  std::vector<HostStage> stages;
  // Masks collected from the op list.
  const uint8_t *row_mask = nullptr, *col_mask = nullptr;
  bool band = false;
  int64_t lo = -kBandNone, hi = kBandNone;
  const int64_t *grow = nullptr, *gcol = nullptr;
  // Batch (pw_bind_batched): B elements; element b reads X + b * sx, Y +
  // b * sy, V + b * sv and each op vector + b * its stride (elements).
  int64_t B = 1, sx = 0, sy = 0, sv = 0;
};

namespace {

// Compute units of the current device (MI355X: 256), read once per device;
// 256 when no device answers (host-only planning, e.g. workspace sizing on a
// machine without a GPU), so a plan never depends on a failed query.
constexpr int kDefaultCUs = 256;
constexpr int kMaxDevices = 64;
int target_cus() {
  static int cached[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = kDefaultCUs;
    }
    __atomic_store_n(&cached[dev], cus, __ATOMIC_RELAXED);
    n = cus;
  }
  return n;
}
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t esize(int dtype) { return dtype == PW_F32 ? 4 : 8; }

struct Plan {
  int family = 0;  // 0: generic VALU engine, 1: MFMA engine
  ValuConfig vcfg{4, 0};
  MfmaConfig mcfg{16, 32, 16};
  int bm = kValuBM, bn = kValuBN;
  int rb_pairs = 0;
  bool order = false;  // pair the row blocks by their dealt tiles (heaviest with lightest)
  size_t off_order = 0;
  size_t off_grp = 0;  // group ranges: rows [n_rb][2], then key tiles [ceil(M / bn)][2]
  size_t off_span = 0;  // kept-tile spans per row block [n_rb][2]
  int n_rb = 0, n_split = 1;
  int n_part = 1;  // partial lists or sums per row the merge reads (0: none)
  int64_t split_cols = 0;
  int chunk = 0;  // value columns per launch (matmul, softmax)
  bool col_norms = false;
  size_t off_epi = 0, off_ny = 0, off_part = 0, part_bytes = 0, total = 0;
  std::vector<size_t> stage_off;  // per stage: offset of its vectors
  // Batched expressions: bytes between consecutive elements' epilogue
  // vectors, column norms and partials (0: shared).
  size_t epi_stride = 0, ny_stride = 0, part_stride = 0;
};

int valu_dtile(int64_t D) { return D <= 3 ? 3 : (D <= 4 ? 4 : (D <= 16 ? 16 : 64)); }
int valu_vtile(int64_t C) { return C <= 4 ? 4 : (C <= 16 ? 16 : 64); }

// The MFMA engine takes D >= 16 (a real contraction) and chains that reduce
// to at most one affine stage with row terms only. For the value consumers
// a narrow V (C < 16) pads the second contraction to 32 (float) or 16
// (double) columns, which only pays once D >= 32.
bool mfma_eligible(const pw_expr &e, int consumer, int64_t C) {
  if (e.D < 16) return false;
  if (e.stages.size() > 1) return false;
  if (e.stages.size() == 1 && (e.stages[0].kind != ST_AFFINE || e.stages[0].col_vec)) return false;
  // Value consumers: the matrix cores take V in columns of 16 or 32, so a
  // narrow V is left to the vector engine unless D is large; a single
  // column (a weighted row sum) is folded with vector FMAs instead.
  if (consumer == PW_C_MATMUL && C == 1) return true;
  if ((consumer == PW_C_MATMUL || consumer == PW_C_SOFTMAX_MATMUL) && C < 16 && e.D < 32) return false;
  return true;
}

Plan make_plan(const pw_expr &e, int consumer, int64_t C, int k) {
  Plan p;
  const size_t es = esize(e.dtype);
  // Epilogue vectors.
  size_t off = 0;
  for (const HostStage &s : e.stages) {
    p.stage_off.push_back(off);
    if (s.kind == ST_AFFINE) {
      if (s.row_vec) off += align_up(2 * (size_t)e.N * es);
      if (s.col_vec) off += align_up(2 * (size_t)e.M * es);
    }
  }
  p.off_epi = 0;
  if (e.B > 1) {  // one set of epilogue vectors per batch element
    p.epi_stride = align_up(off);
    off = p.epi_stride * (size_t)e.B;
  }
  const int cus = target_cus();
  int64_t target_wgs = 4 * (int64_t)cus;
  // The four-rows vector kernels (1024-row blocks, 256-column tiles) only
  // where their grid can still give every CU a workgroup; smaller problems
  // keep the finer-grained kernels.
  const bool four_rows_fill =
      ((e.N + kProdRows * kValuBM - 1) / (kProdRows * kValuBM)) * ((e.M + kProdBN - 1) / kProdBN) >= cus;
  if (mfma_eligible(e, consumer, C)) {
    p.family = 1;
    p.mcfg.dp = e.D <= 16 ? 16 : (e.D <= 32 ? 32 : 64);
    const bool value = consumer == PW_C_MATMUL || consumer == PW_C_SOFTMAX_MATMUL;
    if (!value || (consumer == PW_C_MATMUL && C == 1)) p.mcfg.cp = 1;
    else if (e.dtype == PW_F32) p.mcfg.cp = C <= 32 ? 32 : 64;
    else p.mcfg.cp = C <= 16 ? 16 : (C <= 32 ? 32 : 64);
    p.mcfg.kl = consumer == PW_C_TOPK ? (k <= 16 ? 16 : 64) : 1;
    p.bm = mfma_bm(e.dtype, consumer, p.mcfg.dp, p.mcfg.cp, p.mcfg.kl);
    p.bn = mfma_bn(e.dtype, consumer, p.mcfg.cp, p.mcfg.dp);
    p.chunk = (int)std::min<int64_t>(C, p.mcfg.cp);
    target_wgs = (int64_t)cus * mfma_wgs_per_cu(e.dtype, consumer, p.mcfg.dp, p.mcfg.cp, p.mcfg.kl);
  } else {
    p.vcfg.dtile = valu_dtile(e.D);
    if (consumer == PW_C_MATMUL || consumer == PW_C_SOFTMAX_MATMUL) {
      p.vcfg.vtile = valu_vtile(C);
      p.chunk = (int)std::min<int64_t>(C, p.vcfg.vtile);
      // A plain float product of narrow points and values takes several
      // rows per thread (one LDS broadcast serves them all) and wide tiles.
      if (consumer == PW_C_MATMUL && e.dtype == PW_F32 && e.metric != PW_COSINE && e.stages.empty() &&
          !e.row_mask && !e.col_mask && !e.band && !e.grow && p.vcfg.dtile <= 4 && p.vcfg.vtile == 4 &&
          four_rows_fill) {
        p.vcfg.rows = kProdRows;
        p.bm = kProdRows * kValuBM;
        p.bn = kProdBN;
        target_wgs = (int64_t)kProdWGsPerCU * cus;
      }
    } else if (consumer == PW_C_TOPK) {
      // The list is sized to k: its warm-up insertions (and their cost)
      // scale with its length.
      p.vcfg.vtile = k == 1 ? 1 : (k <= 8 ? 8 : (k <= 16 ? 16 : 64));
      // The plain float row minimum of narrow points takes two rows per
      // thread, as the plain product does.
      if (k == 1 && e.dtype == PW_F32 && e.metric != PW_COSINE && e.stages.empty() && !e.row_mask &&
          !e.col_mask && !e.band && !e.grow && p.vcfg.dtile <= 4) {
        p.vcfg.rows = 2;
        p.bm = 2 * kValuBM;
      }
    } else {
      p.vcfg.vtile = 0;
      // The float row log-sum-exp of narrow points under at most one
      // row-only affine stage takes several rows per thread.
      const bool row_affine = e.stages.empty() || (e.stages.size() == 1 && e.stages[0].kind == ST_AFFINE &&
                                                   !e.stages[0].col_vec);
      if (consumer == PW_C_LOGSUMEXP && e.dtype == PW_F32 && e.metric != PW_COSINE && row_affine && !e.row_mask &&
          !e.col_mask && !e.band && !e.grow && p.vcfg.dtile <= 4) {
        if (e.metric == PW_RBF || !four_rows_fill) {
          p.vcfg.rows = 2;
          p.bm = 2 * kValuBM;
        } else {
          // Dot products and squared distances: four rows per thread, the
          // product's wide tiles and many short workgroups.
          p.vcfg.rows = kProdRows;
          p.bm = kProdRows * kValuBM;
          p.bn = kProdBN;
          target_wgs = (int64_t)kProdWGsPerCU * cus;
        }
      }
    }
  }
  // Column norms: |y_j|^2 for the MFMA engine's distance expansion, 1/|y_j|
  // for cosine on either engine.
  p.col_norms = (p.family == 1 && e.metric != PW_LINEAR) || e.metric == PW_COSINE;
  p.off_ny = off;
  if (p.col_norms) {
    const size_t one = align_up((size_t)e.M * es);
    if (e.B > 1 && e.sy != 0) p.ny_stride = one;  // per element, unless Y is shared
    off += e.B > 1 && e.sy != 0 ? one * (size_t)e.B : one;
  }
  // Tile grid: enough workgroups to fill the chip, splitting the columns
  // when there are too few row blocks.
  p.n_rb = (int)((e.N + p.bm - 1) / p.bm);
  // Pair masks make the work per row block uneven (causal: linear in the
  // block); the MFMA engine then pairs the row blocks r and n_rb - 1 - r and
  // deals each pair's kept tiles evenly to the splits.
  p.rb_pairs = (p.family == 1 && (e.band || e.grow)) ? (p.n_rb + 1) / 2 : 0;
  const int rb_slots = p.rb_pairs ? p.rb_pairs : p.n_rb;
  const int64_t tiles = std::max<int64_t>(1, (e.M + p.bn - 1) / p.bn);
  int64_t want = std::max<int64_t>(1, (target_wgs + rb_slots - 1) / std::max(rb_slots, 1));
  want = std::min(want, tiles);
  const int64_t tiles_per_split = (tiles + want - 1) / want;
  p.split_cols = tiles_per_split * p.bn;
  p.n_split = (int)std::max<int64_t>(1, (e.M + p.split_cols - 1) / p.split_cols);
  // Paired launches deal each pair's tiles to the splits (not column
  // ranges): `want` splits, as long as each gets a few tiles.
  if (p.rb_pairs) p.n_split = (int)std::max<int64_t>(1, std::min<int64_t>(want, 2 * tiles / 4));
  // Group ranges of a same_group mask, and per row block the span of tiles
  // the pair masks keep (with groups: a band alone needs no table).
  if (e.grow) {
    p.off_grp = off;
    const int64_t key_tiles = (e.M + p.bn - 1) / p.bn;
    off += align_up((size_t)(p.n_rb + key_tiles) * 2 * sizeof(int64_t));
  }
  if (e.grow) {
    p.off_span = off;
    off += align_up((size_t)p.n_rb * 2 * sizeof(int64_t));
  }
  // With groups the blocks' tile counts follow the groups (a sawtooth for
  // packed sequences): pair them by count, not by index.
  p.order = p.rb_pairs && e.grow && p.n_rb <= kMaxOrderedBlocks;
  if (p.order) {
    p.off_order = off;
    off += align_up((size_t)p.n_rb * sizeof(int));
  }
  // Partials: one per column split, and for MFMA top-k one per split and
  // lane group.
  p.off_part = off;
  p.n_part = p.n_split;
  if (p.family == 1 && consumer == PW_C_TOPK) p.n_part = p.n_split * mfma_groups(e.dtype);
  if (p.n_part > 1) {
    size_t per_row = 0;
    switch (consumer) {
      case PW_C_MATMUL: per_row = (size_t)p.chunk * es; break;
      case PW_C_DISPLACEMENT: per_row = (size_t)e.D * es; break;
      case PW_C_LOGSUMEXP: per_row = 2 * es; break;
      case PW_C_SOFTMAX_MATMUL: per_row = (size_t)(p.chunk + 2) * es; break;
      case PW_C_TOPK: per_row = (size_t)k * (e.dtype == PW_F32 ? 8 : 16); break;
    }
    p.part_bytes = align_up((size_t)p.n_part * (size_t)e.N * per_row);
    if (e.B > 1) {
      p.part_stride = p.part_bytes;
      p.part_bytes *= (size_t)e.B;
    }
  }
  p.total = p.off_part + p.part_bytes;
  if (p.total) p.total += kAlign;  // room to align the caller's pointer
  return p;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int check_expr(const pw_expr *e) { return e ? PW_OK : PW_ERR_INVALID; }

// Validate a consumer call's common arguments and its workspace.
int check_ws(const Plan &p, void *ws, size_t ws_bytes, char **base) {
  *base = nullptr;
  if (p.total == 0) return PW_OK;
  if (!ws || ws_bytes < p.total) return PW_ERR_WORKSPACE;
  uintptr_t b = ((uintptr_t)ws + kAlign - 1) / kAlign * kAlign;
  *base = reinterpret_cast<char *>(b);
  return PW_OK;
}

int hip_status(hipError_t err) { return err == hipSuccess ? PW_OK : PW_ERR_HIP; }

// Fill the device epilogue and launch the vector programs into the workspace.
int prepare_epilogue(const pw_expr &e, const Plan &p, char *base, Epi *epi, hipStream_t s) {
  std::memset(epi, 0, sizeof(*epi));
  epi->n_stages = (int)e.stages.size();
  VecProgBatch batch;
  std::memset(&batch, 0, sizeof(batch));
  const size_t es = esize(e.dtype);
  auto add_prog = [&](const Prog &pr, void *out, int64_t len) -> int {
    if (len == 0) return PW_OK;
    if (pr.ins.size() > (size_t)kMaxVecInstr) return PW_ERR_UNSUPPORTED;
    VecProg &vp = batch.p[batch.n_progs++];
    vp.n = (int)pr.ins.size();
    vp.len = len;
    vp.out = out;
    vp.out_bstride = (int64_t)p.epi_stride;
    for (size_t t = 0; t < pr.ins.size(); ++t) vp.ins[t] = pr.ins[t];
    if (batch.n_progs == kProgsPerLaunch) {
      int rc = hip_status(launch_vec_progs(e.dtype, batch, e.B, s));
      std::memset(&batch, 0, sizeof(batch));
      return rc;
    }
    return PW_OK;
  };
  for (size_t si = 0; si < e.stages.size(); ++si) {
    const HostStage &hs = e.stages[si];
    Stage &d = epi->st[si];
    d.kind = hs.kind;
    d.row_vec = hs.row_vec;
    d.col_vec = hs.col_vec;
    d.r_scalar = hs.r_scalar;
    d.p_scalar = hs.p_scalar;
    if (hs.kind != ST_AFFINE) continue;
    char *ptr = base + p.off_epi + p.stage_off[si];
    int rc = PW_OK;
    if (hs.row_vec) {
      d.r_vec = ptr;
      d.p_vec = ptr + (size_t)e.N * es;
      rc = add_prog(hs.r, ptr, e.N);
      if (rc == PW_OK) rc = add_prog(hs.p, ptr + (size_t)e.N * es, e.N);
      ptr += align_up(2 * (size_t)e.N * es);
    }
    if (rc == PW_OK && hs.col_vec) {
      epi->any_col = 1;
      d.q_vec = ptr;
      d.o_vec = ptr + (size_t)e.M * es;
      rc = add_prog(hs.q, ptr, e.M);
      if (rc == PW_OK) rc = add_prog(hs.o, ptr + (size_t)e.M * es, e.M);
    }
    if (rc != PW_OK) return rc;
  }
  if (batch.n_progs) return hip_status(launch_vec_progs(e.dtype, batch, e.B, s));
  return PW_OK;
}

TileArgs base_args(const pw_expr &e, const Plan &p, char *base) {
  TileArgs a;
  std::memset(&a, 0, sizeof(a));
  a.X = e.X;
  a.ldx = e.ldx;
  a.Y = e.Y;
  a.ldy = e.ldy;
  a.N = e.N;
  a.M = e.M;
  a.D = (int)e.D;
  a.gamma = e.metric == PW_RBF ? e.gamma : 0.0;
  a.n_rb = p.n_rb;
  a.rb_pairs = p.rb_pairs;
  a.n_split = p.n_split;
  a.split_cols = p.split_cols;
  a.partial = p.n_part > 1 ? base + p.off_part : nullptr;
  a.ny = p.col_norms ? base + p.off_ny : nullptr;
  const int64_t es = (int64_t)esize(e.dtype);
  a.bat.n = e.B;
  a.bat.x = e.sx * es;
  a.bat.y = e.sy * es;
  a.bat.part = (int64_t)p.part_stride;
  a.bat.ny = (int64_t)p.ny_stride;
  a.bat.epi = (int64_t)p.epi_stride;
  // Taylor coefficients of e^(a f) - 1, a = ln2/256, for the double exp2.
  const long double ak = logl(2.0L) / 256.0L;
  long double c = 1.0L;
  for (int k = 1; k <= 4; ++k) {
    c *= ak / (long double)k;
    a.exp2_c[k - 1] = (double)c;
  }
  return a;
}

hipError_t launch_tile(const pw_expr &e, int consumer, const Plan &p, const TileArgs &a, hipStream_t s) {
  if (p.family == 1) {
    if (e.dtype == PW_F32) {
      switch (e.metric) {
        case PW_LINEAR: return mfma_launch_metric<float, M_LINEAR>(consumer, p.mcfg, a, s);
        case PW_SQEUCLIDEAN: return mfma_launch_metric<float, M_SQEUCLIDEAN>(consumer, p.mcfg, a, s);
        case PW_COSINE: return mfma_launch_metric<float, M_COSINE>(consumer, p.mcfg, a, s);
        default: return mfma_launch_metric<float, M_RBF>(consumer, p.mcfg, a, s);
      }
    }
    switch (e.metric) {
      case PW_LINEAR: return mfma_launch_metric<double, M_LINEAR>(consumer, p.mcfg, a, s);
      case PW_SQEUCLIDEAN: return mfma_launch_metric<double, M_SQEUCLIDEAN>(consumer, p.mcfg, a, s);
      case PW_COSINE: return mfma_launch_metric<double, M_COSINE>(consumer, p.mcfg, a, s);
      default: return mfma_launch_metric<double, M_RBF>(consumer, p.mcfg, a, s);
    }
  }
  if (e.dtype == PW_F32) {
    switch (e.metric) {
      case PW_LINEAR: return valu_launch_metric<float, M_LINEAR>(consumer, p.vcfg, a, s);
      case PW_SQEUCLIDEAN: return valu_launch_metric<float, M_SQEUCLIDEAN>(consumer, p.vcfg, a, s);
      case PW_COSINE: return valu_launch_metric<float, M_COSINE>(consumer, p.vcfg, a, s);
      default: return valu_launch_metric<float, M_RBF>(consumer, p.vcfg, a, s);
    }
  }
  switch (e.metric) {
    case PW_LINEAR: return valu_launch_metric<double, M_LINEAR>(consumer, p.vcfg, a, s);
    case PW_SQEUCLIDEAN: return valu_launch_metric<double, M_SQEUCLIDEAN>(consumer, p.vcfg, a, s);
    case PW_COSINE: return valu_launch_metric<double, M_COSINE>(consumer, p.vcfg, a, s);
    default: return valu_launch_metric<double, M_RBF>(consumer, p.vcfg, a, s);
  }
}

// Column norms |y_j|^2 for the MFMA engine's distance expansion.
int prepare_norms(const pw_expr &e, const Plan &p, const TileArgs &a, hipStream_t s) {
  if (!p.col_norms) return PW_OK;
  const bool per = e.B > 1 && e.sy != 0;
  return hip_status(launch_row_norms(e.dtype, e.Y, e.M, e.ldy, (int)e.D, const_cast<void *>(a.ny), s,
                                     e.metric == PW_COSINE, per ? e.B : 1, per ? a.bat.y : 0,
                                     (int64_t)p.ny_stride));
}

// Mask arguments, and the group ranges per row block and key tile.
int prepare_masks(const pw_expr &e, const Plan &p, char *base, TileArgs &a, hipStream_t s) {
  MaskArgs &m = a.mask;
  m.row = e.row_mask;
  m.col = e.col_mask;
  m.band = e.band ? 1 : 0;
  m.lo = e.lo;
  m.hi = e.hi;
  m.grow = e.grow;
  m.gcol = e.gcol;
  m.any = (m.row || m.col || m.band || m.grow) ? 1 : 0;
  int rc = PW_OK;
  if (e.grow) {
    int64_t *rng = reinterpret_cast<int64_t *>(base + p.off_grp);
    m.grow_rng = rng;
    m.gcol_rng = rng + 2 * (size_t)p.n_rb;
    rc = hip_status(launch_group_ranges(e.grow, e.N, p.bm, rng, s));
    if (rc == PW_OK) rc = hip_status(launch_group_ranges(e.gcol, e.M, p.bn, rng + 2 * (size_t)p.n_rb, s));
  }
  if (rc == PW_OK && e.grow) {  // a band alone gives the range in closed form
    int64_t *span = reinterpret_cast<int64_t *>(base + p.off_span);
    rc = hip_status(launch_tile_spans(m, e.N, e.M, p.bm, p.bn, p.n_rb, span, s));
    m.span = span;  // the spans pass itself runs without them
  }
  if (rc == PW_OK && p.order) {
    int *order = reinterpret_cast<int *>(base + p.off_order);
    rc = hip_status(launch_pair_order(m, e.N, e.M, p.bm, p.bn, p.n_rb, order, s));
    a.rb_order = order;
  }
  return rc;
}

// Everything a tile launch reads besides the caller's arrays.
int prepare(const pw_expr &e, const Plan &p, char *base, TileArgs &a, hipStream_t s) {
  int rc = prepare_epilogue(e, p, base, &a.epi, s);
  if (rc == PW_OK) rc = prepare_norms(e, p, a, s);
  if (rc == PW_OK) rc = prepare_masks(e, p, base, a, s);
  return rc;
}

// Caller-owned events recorded around tile launches (pw_set_tile_events).
thread_local hipEvent_t tile_ev_start = nullptr, tile_ev_stop = nullptr;

// One tile launch plus, when the columns are split, the merge.
int run_tiles(const pw_expr &e, int consumer, const Plan &p, TileArgs &a, hipStream_t s, bool first = true,
              bool last = true) {
  if (first && tile_ev_start) (void)hipEventRecord(tile_ev_start, s);
  int rc = hip_status(launch_tile(e, consumer, p, a, s));
  if (last && tile_ev_stop) (void)hipEventRecord(tile_ev_stop, s);
  if (rc == PW_OK && p.n_part > 1) {
    TileArgs m = a;
    m.n_split = p.n_part;
    rc = hip_status(launch_merge(e.dtype, consumer, m, s));
  }
  return rc;
}

}  // namespace

extern "C" {

int pw_set_tile_events(void *start, void *stop) {
  tile_ev_start = (hipEvent_t)start;
  tile_ev_stop = (hipEvent_t)stop;
  return PW_OK;
}

const char *pw_error_string(int code) {
  switch (code) {
    case PW_OK: return "ok";
    case PW_ERR_INVALID: return "invalid argument";
    case PW_ERR_UNSUPPORTED: return "unsupported: outside the fused range";
    case PW_ERR_WORKSPACE: return "workspace missing or too small";
    case PW_ERR_HIP: return "HIP runtime error";
    case PW_ERR_SCRATCH: return "needs more workspace than the static buffer of pw_topk_noalloc holds";
    default: return "unknown status";
  }
}

static int bind_impl(pw_expr **out, int dtype, int metric, double gamma, const void *X, int64_t N, int64_t ldx,
                     const void *Y, int64_t M, int64_t ldy, int64_t D, const pw_op *ops, int n_ops,
                     const pw_batch *batch) {
  if (!out) return PW_ERR_INVALID;
  *out = nullptr;
  const int64_t *op_bstride = batch ? batch->op_stride : nullptr;
  if (batch) {
    if (batch->B < 1 || batch->sx < 0 || batch->sy < 0 || batch->sv < 0) return PW_ERR_INVALID;
    if (batch->B > kMaxBatch) return PW_ERR_UNSUPPORTED;
    for (int t = 0; t < n_ops && t < PW_MAX_OPS; ++t) {
      if (op_bstride[t] < 0) return PW_ERR_INVALID;
      const int k = ops ? ops[t].kind : -1;
      const bool vec = k == PW_OP_ADD_ROWS || k == PW_OP_ADD_COLUMNS || k == PW_OP_WEIGHT_ROWS ||
                       k == PW_OP_WEIGHT_COLUMNS;
      if (!vec && op_bstride[t] != 0) return PW_ERR_UNSUPPORTED;  // masks are shared by the batch
    }
  }
  if (dtype != PW_F32 && dtype != PW_F64) return PW_ERR_INVALID;
  if (metric < PW_LINEAR || metric > PW_COSINE) return PW_ERR_INVALID;
  if (metric == PW_RBF && !(std::isfinite(gamma) && gamma >= 0.0)) return PW_ERR_INVALID;
  if (N < 0 || M < 0 || n_ops < 0) return PW_ERR_INVALID;
  if (D < 1 || D > PW_MAX_D) return PW_ERR_UNSUPPORTED;
  if (N > INT32_MAX || M > INT32_MAX) return PW_ERR_UNSUPPORTED;
  if (ldx < D || ldy < D) return PW_ERR_INVALID;
  const size_t es = esize(dtype);
  if ((N > 0 && !X) || (M > 0 && !Y)) return PW_ERR_INVALID;
  if (!aligned(X, es) || !aligned(Y, es)) return PW_ERR_INVALID;
  if (n_ops > PW_MAX_OPS) return PW_ERR_UNSUPPORTED;
  if (n_ops > 0 && !ops) return PW_ERR_INVALID;
  for (int t = 0; t < n_ops; ++t) {
    const pw_op &o = ops[t];
    switch (o.kind) {
      case PW_OP_MUL:
      case PW_OP_ADD:
        if (!std::isfinite(o.scalar)) return PW_ERR_INVALID;
        break;
      case PW_OP_ADD_ROWS:
      case PW_OP_WEIGHT_ROWS:
        if ((N > 0 && !o.vec) || !aligned(o.vec, es)) return PW_ERR_INVALID;
        break;
      case PW_OP_ADD_COLUMNS:
      case PW_OP_WEIGHT_COLUMNS:
        if ((M > 0 && !o.vec) || !aligned(o.vec, es)) return PW_ERR_INVALID;
        break;
      case PW_OP_EXP: break;
      case PW_OP_MASK_ROWS:
      case PW_OP_GROUP_ROWS:
        if (N > 0 && !o.vec) return PW_ERR_INVALID;
        if (o.kind == PW_OP_GROUP_ROWS && !aligned(o.vec, 8)) return PW_ERR_INVALID;
        break;
      case PW_OP_MASK_COLUMNS:
      case PW_OP_GROUP_COLUMNS:
        if (M > 0 && !o.vec) return PW_ERR_INVALID;
        if (o.kind == PW_OP_GROUP_COLUMNS && !aligned(o.vec, 8)) return PW_ERR_INVALID;
        break;
      case PW_OP_BAND_UPPER:
      case PW_OP_BAND_LOWER:
        if (!(std::fabs(o.scalar) <= 9007199254740992.0) || o.scalar != std::floor(o.scalar))
          return PW_ERR_INVALID;
        break;
      default: return PW_ERR_INVALID;
    }
  }
  int n_kind[16] = {0};
  for (int t = 0; t < n_ops; ++t) n_kind[ops[t].kind]++;
  if (n_kind[PW_OP_MASK_ROWS] > 1 || n_kind[PW_OP_MASK_COLUMNS] > 1 || n_kind[PW_OP_GROUP_ROWS] > 1 ||
      n_kind[PW_OP_GROUP_COLUMNS] > 1 || n_kind[PW_OP_GROUP_ROWS] != n_kind[PW_OP_GROUP_COLUMNS])
    return PW_ERR_INVALID;
  pw_expr *e = new (std::nothrow) pw_expr();
  if (!e) return PW_ERR_INVALID;
  e->dtype = dtype;
  e->metric = metric;
  e->gamma = gamma;
  e->X = X;
  e->N = N;
  e->ldx = ldx;
  e->Y = Y;
  e->M = M;
  e->ldy = ldy;
  e->D = D;
  e->ops.assign(ops, ops + n_ops);
  for (const pw_op &o : e->ops) {
    switch (o.kind) {
      case PW_OP_MASK_ROWS: e->row_mask = static_cast<const uint8_t *>(o.vec); break;
      case PW_OP_MASK_COLUMNS: e->col_mask = static_cast<const uint8_t *>(o.vec); break;
      case PW_OP_GROUP_ROWS: e->grow = static_cast<const int64_t *>(o.vec); break;
      case PW_OP_GROUP_COLUMNS: e->gcol = static_cast<const int64_t *>(o.vec); break;
      case PW_OP_BAND_UPPER:
        e->band = true;
        e->hi = std::min(e->hi, (int64_t)o.scalar);
        break;
      case PW_OP_BAND_LOWER:
        e->band = true;
        e->lo = std::max(e->lo, -(int64_t)o.scalar);
        break;
    }
  }
  // Bounds beyond the matrix mean the same as none, and keep the device
  // arithmetic on them free of overflow.
  e->hi = std::max(std::min(e->hi, kBandNone), -kBandNone);
  e->lo = std::max(std::min(e->lo, kBandNone), -kBandNone);
  StageBuilder b;
  for (size_t t = 0; t < e->ops.size(); ++t) b.op(e->ops[t], op_bstride ? op_bstride[t] * (int64_t)es : 0);
  b.close();
  e->stages = b.out;
  if (e->stages.size() > (size_t)kMaxStages) {
    delete e;
    return PW_ERR_UNSUPPORTED;
  }
  if (batch) {
    e->B = batch->B;
    e->sx = batch->sx;
    e->sy = batch->sy;
    e->sv = batch->sv;
  }
  *out = e;
  return PW_OK;
}

int pw_bind(pw_expr **out, int dtype, int metric, double gamma, const void *X, int64_t N, int64_t ldx,
            const void *Y, int64_t M, int64_t ldy, int64_t D, const pw_op *ops, int n_ops) {
  return bind_impl(out, dtype, metric, gamma, X, N, ldx, Y, M, ldy, D, ops, n_ops, nullptr);
}

int pw_bind_batched(pw_expr **out, int dtype, int metric, double gamma, const void *X, int64_t N, int64_t ldx,
                    const void *Y, int64_t M, int64_t ldy, int64_t D, const pw_op *ops, int n_ops,
                    const pw_batch *batch) {
  if (!batch) return PW_ERR_INVALID;
  return bind_impl(out, dtype, metric, gamma, X, N, ldx, Y, M, ldy, D, ops, n_ops, batch);
}

void pw_release(pw_expr *e) { delete e; }

static int check_consumer_args(const pw_expr *e, int consumer, int64_t C, int k) {
  if (!e) return PW_ERR_INVALID;
  switch (consumer) {
    case PW_C_MATMUL:
    case PW_C_SOFTMAX_MATMUL:
      if (C < 1) return PW_ERR_INVALID;
      return PW_OK;
    case PW_C_DISPLACEMENT:
    case PW_C_LOGSUMEXP:
      return PW_OK;
    case PW_C_TOPK:
      if (k < 0 || k > e->M) return PW_ERR_INVALID;
      if (k > PW_MAX_K) return PW_ERR_UNSUPPORTED;
      return PW_OK;
  }
  return PW_ERR_INVALID;
}

int pw_workspace_size(const pw_expr *e, int consumer, int64_t C, int k, size_t *bytes) {
  if (!bytes) return PW_ERR_INVALID;
  *bytes = 0;
  int rc = check_consumer_args(e, consumer, C, k);
  if (rc != PW_OK) return rc;
  if (e->N == 0 || e->M == 0 || (consumer == PW_C_TOPK && k == 0)) return PW_OK;
  *bytes = make_plan(*e, consumer, C, k).total;
  return PW_OK;
}

int pw_plan_describe(const pw_expr *e, int consumer, int64_t C, int k, char *buf, size_t len) {
  if (!buf || len == 0) return PW_ERR_INVALID;
  int rc = check_consumer_args(e, consumer, C, k);
  if (rc != PW_OK) return rc;
  Plan p = make_plan(*e, consumer, C, k);
  if (p.family == 1)
    std::snprintf(buf, len,
                  "family=mfma dp=%d cp=%d kl=%d bm=%d bn=%d row_blocks=%d row_block_pairs=%d splits=%d partials=%d "
                  "split_cols=%lld stages=%d batch=%lld workspace=%zu",
                  p.mcfg.dp, p.mcfg.cp, p.mcfg.kl, p.bm, p.bn, p.n_rb, p.rb_pairs, p.n_split, p.n_part,
                  (long long)p.split_cols, (int)e->stages.size(), (long long)e->B, p.total);
  else
    std::snprintf(buf, len,
                  "family=valu dtile=%d vtile=%d rows=%d bm=%d bn=%d row_blocks=%d splits=%d split_cols=%lld stages=%d "
                  "batch=%lld workspace=%zu",
                  p.vcfg.dtile, p.vcfg.vtile, p.vcfg.rows, p.bm, p.bn, p.n_rb, p.n_split, (long long)p.split_cols,
                  (int)e->stages.size(), (long long)e->B, p.total);
  return PW_OK;
}

// Shared body of the value-matrix consumers (matmul, softmax).
static int value_consumer(const pw_expr *e, int consumer, const void *V, int64_t C, int64_t ldv, void *out,
                          int64_t ldo, void *ws, size_t ws_bytes, void *stream, void *lse_out = nullptr) {
  int rc = check_consumer_args(e, consumer, C, 0);
  if (rc != PW_OK) return rc;
  const size_t es = esize(e->dtype);
  if (ldv < C || ldo < C) return PW_ERR_INVALID;
  if ((e->M > 0 && !V) || (e->N > 0 && !out)) return PW_ERR_INVALID;
  if (!aligned(V, es) || !aligned(out, es)) return PW_ERR_INVALID;
  if (lse_out && !aligned(lse_out, es)) return PW_ERR_INVALID;
  if (e->N == 0) return PW_OK;
  hipStream_t s = (hipStream_t)stream;
  if (e->M == 0) {  // batched outputs are packed: B * N rows
    rc = hip_status(launch_fill(e->dtype, out, e->B * e->N, C, ldo, 0.0, s));
    if (rc == PW_OK && lse_out) rc = hip_status(launch_fill(e->dtype, lse_out, e->B * e->N, 1, 1, -HUGE_VAL, s));
    return rc;
  }
  Plan p = make_plan(*e, consumer, C, 0);
  char *base;
  rc = check_ws(p, ws, ws_bytes, &base);
  if (rc != PW_OK) return rc;
  TileArgs a = base_args(*e, p, base);
  rc = prepare(*e, p, base, a, s);
  if (rc != PW_OK) return rc;
  a.ldv = ldv;
  a.ldo = ldo;
  a.lse_out = consumer == PW_C_SOFTMAX_MATMUL ? lse_out : nullptr;
  a.bat.out = e->N * ldo * (int64_t)es;
  a.bat.lse = a.lse_out ? e->N * (int64_t)es : 0;
  a.bat.v = e->sv * (int64_t)es;
  const int cons = consumer == PW_C_MATMUL ? C_MATMUL : C_SOFTMAX;
  for (int64_t c0 = 0; c0 < C && rc == PW_OK; c0 += p.chunk) {
    a.C = (int)std::min<int64_t>(p.chunk, C - c0);
    a.V = static_cast<const char *>(V) + c0 * es;
    a.out = static_cast<char *>(out) + c0 * es;
    rc = run_tiles(*e, cons, p, a, s, c0 == 0, c0 + p.chunk >= C);
  }
  return rc;
}

int pw_matmul(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *ws,
              size_t ws_bytes, void *stream) {
  return value_consumer(e, PW_C_MATMUL, V, C, ldv, out, ldo, ws, ws_bytes, stream);
}

int pw_softmax_matmul(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *ws,
                      size_t ws_bytes, void *stream) {
  return value_consumer(e, PW_C_SOFTMAX_MATMUL, V, C, ldv, out, ldo, ws, ws_bytes, stream);
}

int pw_softmax_matmul_lse(const pw_expr *e, const void *V, int64_t C, int64_t ldv, void *out, int64_t ldo, void *lse,
                          void *ws, size_t ws_bytes, void *stream) {
  if (e && e->N > 0 && !lse) return PW_ERR_INVALID;
  return value_consumer(e, PW_C_SOFTMAX_MATMUL, V, C, ldv, out, ldo, ws, ws_bytes, stream, lse);
}

int pw_displacement(const pw_expr *e, void *out, int64_t ldo, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_consumer_args(e, PW_C_DISPLACEMENT, 0, 0);
  if (rc != PW_OK) return rc;
  if (ldo < e->D || (e->N > 0 && !out) || !aligned(out, esize(e->dtype))) return PW_ERR_INVALID;
  if (e->N == 0) return PW_OK;
  hipStream_t s = (hipStream_t)stream;
  if (e->M == 0) return hip_status(launch_fill(e->dtype, out, e->B * e->N, e->D, ldo, 0.0, s));
  Plan p = make_plan(*e, PW_C_DISPLACEMENT, 0, 0);
  char *base;
  rc = check_ws(p, ws, ws_bytes, &base);
  if (rc != PW_OK) return rc;
  TileArgs a = base_args(*e, p, base);
  rc = prepare(*e, p, base, a, s);
  if (rc != PW_OK) return rc;
  a.out = out;
  a.ldo = ldo;
  a.bat.out = e->N * ldo * (int64_t)esize(e->dtype);
  return run_tiles(*e, C_DISPLACEMENT, p, a, s);
}

int pw_logsumexp(const pw_expr *e, int exclude_self, void *out, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_consumer_args(e, PW_C_LOGSUMEXP, 0, 0);
  if (rc != PW_OK) return rc;
  if (exclude_self != 0 && exclude_self != 1) return PW_ERR_INVALID;
  if ((e->N > 0 && !out) || !aligned(out, esize(e->dtype))) return PW_ERR_INVALID;
  if (e->N == 0) return PW_OK;
  hipStream_t s = (hipStream_t)stream;
  if (e->M == 0) return hip_status(launch_fill(e->dtype, out, e->B * e->N, 1, 1, -HUGE_VAL, s));
  Plan p = make_plan(*e, PW_C_LOGSUMEXP, 0, 0);
  char *base;
  rc = check_ws(p, ws, ws_bytes, &base);
  if (rc != PW_OK) return rc;
  TileArgs a = base_args(*e, p, base);
  rc = prepare(*e, p, base, a, s);
  if (rc != PW_OK) return rc;
  a.out = out;
  a.exclude_self = exclude_self;
  a.bat.out = e->N * (int64_t)esize(e->dtype);
  return run_tiles(*e, C_LOGSUMEXP, p, a, s);
}

int pw_topk(const pw_expr *e, int k, int largest, void *values, int64_t *indices, void *ws, size_t ws_bytes,
            void *stream) {
  int rc = check_consumer_args(e, PW_C_TOPK, 0, k);
  if (rc != PW_OK) return rc;
  if (largest != 0 && largest != 1) return PW_ERR_INVALID;
  if (e->N == 0 || k == 0) return PW_OK;
  if (!values || !indices || !aligned(values, esize(e->dtype)) || !aligned(indices, 8)) return PW_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;
  Plan p = make_plan(*e, PW_C_TOPK, 0, k);
  char *base;
  rc = check_ws(p, ws, ws_bytes, &base);
  if (rc != PW_OK) return rc;
  TileArgs a = base_args(*e, p, base);
  rc = prepare(*e, p, base, a, s);
  if (rc != PW_OK) return rc;
  a.out = values;
  a.idx = indices;
  a.k = k;
  a.largest = largest;
  a.bat.out = e->N * k * (int64_t)esize(e->dtype);
  a.bat.idx = e->N * k * (int64_t)sizeof(int64_t);
  return run_tiles(*e, C_TOPK, p, a, s);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Row means: the kernel product with a column of ones, divided by each
// row's kept count. Without masks the count is M. With masks it is a second
// product over the same masks whose every pair scores 1: the linear metric
// of one-feature points that are all 1, so no input value can overflow it.
// ---------------------------------------------------------------------------
namespace {

bool is_mask_op(int kind) {
  return kind == PW_OP_MASK_ROWS || kind == PW_OP_MASK_COLUMNS || kind == PW_OP_GROUP_ROWS ||
         kind == PW_OP_GROUP_COLUMNS || kind == PW_OP_BAND_UPPER || kind == PW_OP_BAND_LOWER;
}

struct ExprHolder {
  pw_expr *e = nullptr;
  ~ExprHolder() { delete e; }
};

// The unit-score count expression of e over `ones` (>= max(N, M) entries),
// or none when e has no masks. Unbatched: masks are shared by the batch.
int count_expr(const pw_expr &e, const void *ones, ExprHolder *out) {
  std::vector<pw_op> masks;
  for (const pw_op &o : e.ops)
    if (is_mask_op(o.kind)) masks.push_back(o);
  if (masks.empty()) return PW_OK;
  return bind_impl(&out->e, e.dtype, PW_LINEAR, 1.0, ones, e.N, 1, ones, e.M, 1, 1, masks.data(), (int)masks.size(),
                   nullptr);
}

// Workspace of a mean: ones [max(N, M)], counts [N], then the products'
// workspace (the larger of the two).
struct MeanLayout {
  size_t cnt = 0, prod = 0, prod_bytes = 0, total = 0;
};

MeanLayout mean_layout(const pw_expr &e, const pw_expr *ce) {
  MeanLayout L;
  const size_t es = esize(e.dtype);
  size_t off = align_up((size_t)std::max(e.N, e.M) * es);
  L.cnt = off;
  off += align_up((size_t)e.N * es);
  L.prod = off;
  L.prod_bytes = make_plan(e, PW_C_MATMUL, 1, 0).total;
  if (ce) L.prod_bytes = std::max(L.prod_bytes, make_plan(*ce, PW_C_MATMUL, 1, 0).total);
  L.total = off + L.prod_bytes + kAlign;
  return L;
}

}  // namespace

extern "C" {

int pw_mean_workspace_size(const pw_expr *e, size_t *bytes) {
  if (!e || !bytes) return PW_ERR_INVALID;
  *bytes = 0;
  if (e->N == 0 || e->M == 0) return PW_OK;
  ExprHolder ce;
  // Only sizes matter here: any aligned non-null pointer stands for the ones.
  int rc = count_expr(*e, reinterpret_cast<const void *>(kAlign), &ce);
  if (rc != PW_OK) return rc;
  *bytes = mean_layout(*e, ce.e).total;
  return PW_OK;
}

int pw_mean(const pw_expr *e, void *out, void *inv_counts, void *ws, size_t ws_bytes, void *stream) {
  if (!e) return PW_ERR_INVALID;
  const size_t es = esize(e->dtype);
  if ((e->N > 0 && !out) || !aligned(out, es) || !aligned(inv_counts, es)) return PW_ERR_INVALID;
  if (e->N == 0) return PW_OK;
  hipStream_t s = (hipStream_t)stream;
  if (e->M == 0) {  // no kept pair anywhere: NaN means, zero inverse counts
    int rc = hip_status(launch_fill(e->dtype, out, e->B * e->N, 1, 1, 0.0, s));
    if (rc == PW_OK) rc = hip_status(launch_mean_finish(e->dtype, out, e->N, e->B, nullptr, 0, inv_counts, s));
    return rc;
  }
  ExprHolder ce;
  int rc = count_expr(*e, reinterpret_cast<const void *>(kAlign), &ce);
  if (rc != PW_OK) return rc;
  const MeanLayout L = mean_layout(*e, ce.e);
  if (!ws || ws_bytes < L.total) return PW_ERR_WORKSPACE;
  char *base = reinterpret_cast<char *>(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
  void *ones = base, *cnt = base + L.cnt;
  rc = hip_status(launch_fill(e->dtype, ones, std::max(e->N, e->M), 1, 1, 1.0, s));
  pw_expr sums = *e;
  sums.sv = 0;  // the column of ones is shared by the batch
  if (rc == PW_OK) rc = value_consumer(&sums, PW_C_MATMUL, ones, 1, 1, out, 1, base + L.prod, L.prod_bytes, stream);
  if (rc == PW_OK && ce.e) {
    ce.e->X = ones;
    ce.e->Y = ones;
    rc = value_consumer(ce.e, PW_C_MATMUL, ones, 1, 1, cnt, 1, base + L.prod, L.prod_bytes, stream);
  }
  if (rc == PW_OK)
    rc = hip_status(launch_mean_finish(e->dtype, out, e->N, e->B, ce.e ? cnt : nullptr, e->M, inv_counts, s));
  return rc;
}

}  // extern "C"

// ------------------------------------------------------------------ backward

namespace {

constexpr int kGradRows = 256, kGradCols = 64;  // grad_tile workgroup rows and tile

int grad_dtile(int64_t D) { return D <= 4 ? 4 : (D <= 16 ? 16 : 64); }
bool is_vec_op(int kind) {
  return kind == PW_OP_ADD_ROWS || kind == PW_OP_ADD_COLUMNS || kind == PW_OP_WEIGHT_ROWS ||
         kind == PW_OP_WEIGHT_COLUMNS;
}
bool is_arith_op(int kind) { return kind >= PW_OP_MUL && kind <= PW_OP_EXP; }

struct GradPlan {
  int dt = 4, ct = 16, n_arith = 0;
  int n_rb[2] = {0, 0}, n_split[2] = {1, 1}, W[2] = {0, 0};
  int64_t split[2] = {0, 0};
  // The matrix-core backward (128-row workgroups, two per CU).
  int m_n_rb[2] = {0, 0}, m_n_split[2] = {1, 1}, m_pairs[2] = {0, 0};
  int64_t m_split[2] = {0, 0};
  size_t off_lse = 0, off_delta = 0, off_invx = 0, off_invy = 0, off_part = 0, off_fwd = 0, off_epi = 0, total = 0;
};

GradPlan grad_plan(const pw_expr &e, int consumer, int64_t C) {
  GradPlan g;
  const size_t es = esize(e.dtype);
  g.dt = grad_dtile(e.D);
  g.ct = C <= 16 ? 16 : 64;
  for (const pw_op &o : e.ops) g.n_arith += is_arith_op(o.kind);
  const bool value = consumer == PW_C_MATMUL || consumer == PW_C_SOFTMAX_MATMUL;
  const int cus = target_cus();
  size_t part = 0;
  for (int side = 0; side < 2; ++side) {
    const int64_t n_own = side == 0 ? e.N : e.M, n_oth = side == 0 ? e.M : e.N;
    g.n_rb[side] = (int)std::max<int64_t>(1, (n_own + kGradRows - 1) / kGradRows);
    const int64_t tiles = std::max<int64_t>(1, (n_oth + kGradCols - 1) / kGradCols);
    int64_t want = std::max<int64_t>(1, (4 * (int64_t)cus + g.n_rb[side] - 1) / g.n_rb[side]);
    want = std::min(want, tiles);
    g.split[side] = (tiles + want - 1) / want * kGradCols;
    g.n_split[side] = (int)std::max<int64_t>(1, (n_oth + g.split[side] - 1) / g.split[side]);
    g.W[side] = (int)e.D + ((side == 1 && value) ? (int)C : 0) + g.n_arith;
    part = std::max(part, (size_t)g.n_split[side] * (size_t)n_own * (size_t)g.W[side] * es);
    const int mrows = mfma_grad_rows();
    g.m_n_rb[side] = (int)std::max<int64_t>(1, (n_own + mrows - 1) / mrows);
    int64_t mwant = std::max<int64_t>(1, (2 * (int64_t)cus + g.m_n_rb[side] - 1) / g.m_n_rb[side]);
    mwant = std::min(mwant, tiles);
    g.m_split[side] = (tiles + mwant - 1) / mwant * kGradCols;
    g.m_n_split[side] = (int)std::max<int64_t>(1, (n_oth + g.m_split[side] - 1) / g.m_split[side]);
    if (e.band) {  // paired blocks: a pair's band tiles are dealt to the splits
      g.m_pairs[side] = (g.m_n_rb[side] + 1) / 2;
      const int64_t pw_ = std::max<int64_t>(1, (2 * (int64_t)cus + g.m_pairs[side] - 1) / g.m_pairs[side]);
      g.m_n_split[side] = (int)std::max<int64_t>(1, std::min<int64_t>(pw_, 2 * tiles / 4));
    }
    part = std::max(part, (size_t)g.m_n_split[side] * (size_t)n_own * (size_t)g.W[side] * es);
  }
  size_t off = 0;
  g.off_lse = off;
  off += align_up((size_t)e.N * es);
  g.off_delta = off;
  off += align_up((size_t)e.N * es);
  g.off_invx = off;
  off += align_up((size_t)e.N * es);
  g.off_invy = off;
  off += align_up((size_t)e.M * es);
  g.off_part = off;
  off += align_up(part);
  g.off_fwd = off;
  if (consumer == PW_C_LOGSUMEXP || consumer == PW_C_SOFTMAX_MATMUL) off += align_up(make_plan(e, PW_C_LOGSUMEXP, 0, 0).total);
  // The canonical stage's vectors for the fast path (the forward's layout).
  g.off_epi = off;
  off += align_up(make_plan(e, PW_C_MATMUL, 1, 0).off_ny);
  g.total = off + kAlign;
  return g;
}

}  // namespace

extern "C" {

int pw_backward_plan_describe(const pw_expr *e, int consumer, int64_t C, int want_ops, char *buf, size_t len) {
  if (!e || !buf || len == 0 || consumer < PW_C_MATMUL || consumer > PW_C_TOPK) return PW_ERR_INVALID;
  if (e->B > 1) return PW_ERR_UNSUPPORTED;  // the backward runs per batch element
  const GradPlan g = grad_plan(*e, consumer, std::max<int64_t>(C, 1));
  const bool fast = !want_ops && e->stages.size() <= 1 && (e->stages.empty() || e->stages[0].kind == ST_AFFINE);
  const bool col_stage = !e->stages.empty() && e->stages[0].col_vec;
  const bool mfma = e->dtype == PW_F32 && e->metric == PW_LINEAR && fast && !col_stage && !e->grow && e->D >= 16 &&
                    (consumer == PW_C_SOFTMAX_MATMUL || consumer == PW_C_LOGSUMEXP);
  if (consumer == PW_C_TOPK)
    std::snprintf(buf, len, "family=grad_topk dtile=%d", g.dt);
  else if (mfma)
    std::snprintf(buf, len, "family=mfma_grad dp=%d cp=%d rows_per_wg=%d splits=%d/%d", e->D <= 16 ? 16 : (e->D <= 32 ? 32 : 64),
                  C <= 32 ? 32 : 64, mfma_grad_rows(), g.m_n_split[0], g.m_n_split[1]);
  else
    std::snprintf(buf, len, "family=valu_grad dtile=%d ctile=%d fast=%d splits=%d/%d", g.dt, g.ct, fast ? 1 : 0,
                  g.n_split[0], g.n_split[1]);
  return PW_OK;
}

int pw_backward_workspace_size(const pw_expr *e, int consumer, int64_t C, int k, size_t *bytes) {
  (void)k;
  if (!e || !bytes || consumer < PW_C_MATMUL || consumer > PW_C_TOPK) return PW_ERR_INVALID;
  if (e->B > 1) return PW_ERR_UNSUPPORTED;
  *bytes = grad_plan(*e, consumer, std::max<int64_t>(C, 1)).total;
  return PW_OK;
}

int pw_backward(const pw_expr *e, int consumer, const pw_grad_in *in, const pw_grad_out *out, void *ws,
                size_t ws_bytes, void *stream) {
  if (!e || !in || !out || consumer < PW_C_MATMUL || consumer > PW_C_TOPK) return PW_ERR_INVALID;
  if (e->B > 1) return PW_ERR_UNSUPPORTED;
  const size_t es = esize(e->dtype);
  const bool value = consumer == PW_C_MATMUL || consumer == PW_C_SOFTMAX_MATMUL;
  const int64_t C = value ? in->C : 0;
  if (value) {
    if (C < 1) return PW_ERR_INVALID;
    if (C > 64) return PW_ERR_UNSUPPORTED;
    if ((e->M > 0 && !in->V) || in->ldv < C || in->ldg < C || !aligned(in->V, es)) return PW_ERR_INVALID;
  }
  if (consumer == PW_C_SOFTMAX_MATMUL &&
      ((e->N > 0 && !in->out) || in->ldo < C || !aligned(in->out, es) || !aligned(in->lse, es)))
    return PW_ERR_INVALID;
  if (consumer == PW_C_DISPLACEMENT && in->ldg < e->D) return PW_ERR_INVALID;
  if (consumer == PW_C_LOGSUMEXP && (in->ldg < 1 || (in->exclude_self != 0 && in->exclude_self != 1) ||
                                     !aligned(in->out, es)))
    return PW_ERR_INVALID;
  if (consumer == PW_C_TOPK) {
    if (in->k < 1 || in->k > e->M || in->ldg < in->k || (e->N > 0 && !in->indices) || !aligned(in->indices, 8))
      return PW_ERR_INVALID;
    if (in->k > PW_MAX_K) return PW_ERR_UNSUPPORTED;
  }
  if ((e->N > 0 && !in->G) || !aligned(in->G, es)) return PW_ERR_INVALID;
  if ((out->dX && (out->lddx < e->D || !aligned(out->dX, es))) ||
      (out->dY && (out->lddy < e->D || !aligned(out->dY, es))) ||
      (out->dV && (!value || out->lddv < C || !aligned(out->dV, es))))
    return PW_ERR_INVALID;
  for (size_t t = 0; t < e->ops.size(); ++t)
    if (out->dops[t] && !aligned(out->dops[t], es)) return PW_ERR_INVALID;
  hipStream_t s = (hipStream_t)stream;

  // Arithmetic ops in order, and for each the caller's output slot.
  GradArgs a;
  std::memset(&a, 0, sizeof(a));
  int bound_of[kGradOps];
  for (size_t t = 0; t < e->ops.size(); ++t) {
    const pw_op &o = e->ops[t];
    if (!is_arith_op(o.kind)) continue;
    GradOp &g = a.ops[a.n_ops];
    g.kind = o.kind;
    g.scalar = o.scalar;
    g.vec = o.vec;
    g.where = (o.kind == PW_OP_ADD_ROWS || o.kind == PW_OP_WEIGHT_ROWS) ? 1
              : (o.kind == PW_OP_ADD_COLUMNS || o.kind == PW_OP_WEIGHT_COLUMNS) ? 2 : 0;
    bound_of[a.n_ops++] = (int)t;
  }
  auto want_side = [&](int side) {
    if (side == 0 ? out->dX != nullptr : (out->dY != nullptr || out->dV != nullptr)) return true;
    for (int t = 0; t < a.n_ops; ++t)
      if (a.ops[t].where == side + 1 && out->dops[bound_of[t]]) return true;
    return false;
  };

  // Empty sets: every requested gradient is zero.
  if (e->N == 0 || e->M == 0) {
    int rc = PW_OK;
    if (out->dX && rc == PW_OK) rc = hip_status(launch_fill(e->dtype, out->dX, e->N, e->D, out->lddx, 0.0, s));
    if (out->dY && rc == PW_OK) rc = hip_status(launch_fill(e->dtype, out->dY, e->M, e->D, out->lddy, 0.0, s));
    if (out->dV && rc == PW_OK) rc = hip_status(launch_fill(e->dtype, out->dV, e->M, C, out->lddv, 0.0, s));
    for (int t = 0; t < a.n_ops && rc == PW_OK; ++t)
      if (a.ops[t].where && out->dops[bound_of[t]])
        rc = hip_status(launch_fill(e->dtype, out->dops[bound_of[t]], a.ops[t].where == 1 ? e->N : e->M, 1, 1,
                                    0.0, s));
    return rc;
  }

  const GradPlan g = grad_plan(*e, consumer, std::max<int64_t>(C, 1));
  if (!ws || ws_bytes < g.total) return PW_ERR_WORKSPACE;
  char *base = reinterpret_cast<char *>(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
  a.X = e->X;
  a.Y = e->Y;
  a.ldx = e->ldx;
  a.ldy = e->ldy;
  a.N = e->N;
  a.M = e->M;
  a.D = (int)e->D;
  a.gamma = e->metric == PW_RBF ? e->gamma : 0.0;
  a.G = in->G;
  a.ldg = in->ldg;
  a.V = in->V;
  a.ldv = in->ldv;
  a.C = (int)C;
  a.exclude_self = consumer == PW_C_LOGSUMEXP ? in->exclude_self : 0;
  a.mask.row = e->row_mask;
  a.mask.col = e->col_mask;
  a.mask.band = e->band ? 1 : 0;
  a.mask.lo = e->lo;
  a.mask.hi = e->hi;
  a.mask.grow = e->grow;
  a.mask.gcol = e->gcol;
  a.mask.any = (a.mask.row || a.mask.col || a.mask.band || a.mask.grow) ? 1 : 0;
  int rc = PW_OK;
  if (e->metric == PW_COSINE) {
    a.inv_x = base + g.off_invx;
    a.inv_y = base + g.off_invy;
    rc = hip_status(launch_row_norms(e->dtype, e->X, e->N, e->ldx, (int)e->D, base + g.off_invx, s, true));
    if (rc == PW_OK)
      rc = hip_status(launch_row_norms(e->dtype, e->Y, e->M, e->ldy, (int)e->D, base + g.off_invy, s, true));
  }
  if (rc == PW_OK && (consumer == PW_C_LOGSUMEXP || consumer == PW_C_SOFTMAX_MATMUL)) {
    if (consumer == PW_C_LOGSUMEXP && in->out) {
      a.lse = in->out;
    } else if (consumer == PW_C_SOFTMAX_MATMUL && in->lse) {
      a.lse = in->lse;
    } else {
      // The row log-sum-exp of the forward scores: one more forward pass.
      a.lse = base + g.off_lse;
      const size_t fwd = make_plan(*e, PW_C_LOGSUMEXP, 0, 0).total;
      rc = pw_logsumexp(e, a.exclude_self, base + g.off_lse, base + g.off_fwd, fwd, stream);
    }
    if (rc == PW_OK && consumer == PW_C_SOFTMAX_MATMUL) {
      a.delta = base + g.off_delta;
      rc = hip_status(launch_grad_delta(e->dtype, in->G, in->ldg, in->out, in->ldo, e->N, (int)C,
                                        base + g.off_delta, s));
    }
  }
  if (rc != PW_OK) return rc;

  if (consumer == PW_C_TOPK) {
    a.idx = in->indices;
    a.k = in->k;
    a.dX = out->dX;
    a.dY = out->dY;
    a.lddx = out->lddx;
    a.lddy = out->lddy;
    for (int t = 0; t < a.n_ops; ++t) a.dop[t] = out->dops[bound_of[t]];
    // Column-side results are summed atomically into cleared outputs.
    if (out->dY) rc = hip_status(launch_fill(e->dtype, out->dY, e->M, e->D, out->lddy, 0.0, s));
    for (int t = 0; t < a.n_ops && rc == PW_OK; ++t)
      if (a.ops[t].where == 2 && a.dop[t]) rc = hip_status(launch_fill(e->dtype, a.dop[t], e->M, 1, 1, 0.0, s));
    if (rc == PW_OK) rc = hip_status(grad_topk_launch(e->dtype, e->metric, g.dt, a, s));
    return rc;
  }

  // Fast path: the ops fold into at most one affine stage and no op-vector
  // gradient is wanted; the stage's vectors come from the forward's own
  // pre-pass.
  bool want_ops = false;
  for (int t = 0; t < a.n_ops; ++t) want_ops |= a.ops[t].where && out->dops[bound_of[t]] != nullptr;
  if (!want_ops && e->stages.size() <= 1 && (e->stages.empty() || e->stages[0].kind == ST_AFFINE)) {
    a.fast = 1;
    Epi epi;
    Plan ep = make_plan(*e, PW_C_MATMUL, 1, 0);
    rc = prepare_epilogue(*e, ep, base + g.off_epi, &epi, s);
    if (rc != PW_OK) return rc;
    if (epi.n_stages == 1) {
      a.stage = epi.st[0];
    } else {
      std::memset(&a.stage, 0, sizeof(a.stage));
      a.stage.kind = ST_AFFINE;
      a.stage.r_scalar = 1.0;
    }
  }
  const int cons = consumer == PW_C_MATMUL ? C_MATMUL
                   : consumer == PW_C_DISPLACEMENT ? C_DISPLACEMENT
                   : consumer == PW_C_LOGSUMEXP ? C_LOGSUMEXP : C_SOFTMAX;
  const int last_side = want_side(1) ? 1 : 0;
  bool started = false;

  // Dot-product scores with one row-only affine stage, float32, no masks:
  // the matrix-core backward (softmax@V and logsumexp).
  const bool mfma = e->dtype == PW_F32 && e->metric == PW_LINEAR && a.fast && !a.stage.col_vec && !a.mask.grow &&
                    e->D >= 16 && (cons == C_SOFTMAX || cons == C_LOGSUMEXP);
  if (mfma) {
    MfmaGradArgs m;
    std::memset(&m, 0, sizeof(m));
    m.X = static_cast<const float *>(e->X);
    m.Y = static_cast<const float *>(e->Y);
    m.V = static_cast<const float *>(in->V);
    m.G = static_cast<const float *>(in->G);
    m.ldx = e->ldx;
    m.ldy = e->ldy;
    m.ldv = in->ldv;
    m.ldg = in->ldg;
    m.N = e->N;
    m.M = e->M;
    m.D = (int)e->D;
    m.C = (int)C;
    m.lse = static_cast<const float *>(a.lse);
    m.delta = static_cast<const float *>(a.delta);
    m.row_vec = a.stage.row_vec;
    m.r_s = (float)a.stage.r_scalar;
    m.p_s = (float)a.stage.p_scalar;
    m.r_vec = static_cast<const float *>(a.stage.r_vec);
    m.p_vec = static_cast<const float *>(a.stage.p_vec);
    m.exclude_self = a.exclude_self;
    m.mask = a.mask;
    m.partial = reinterpret_cast<float *>(base + g.off_part);
    const int dp = e->D <= 16 ? 16 : (e->D <= 32 ? 32 : 64);
    const int cp = C <= 32 ? 32 : 64;
    for (int side = 0; side < 2 && rc == PW_OK; ++side) {
      if (!want_side(side)) continue;
      if (!started && tile_ev_start) (void)hipEventRecord(tile_ev_start, s);
      started = true;
      m.n_rb = g.m_n_rb[side];
      m.n_split = g.m_n_split[side];
      m.split = g.m_split[side];
      m.rb_pairs = g.m_pairs[side];
      m.W = (int)e->D + ((side == 1 && cons == C_SOFTMAX) ? (int)C : 0);
      rc = hip_status(mfma_grad_launch(cons, side, dp, cp, m, s));
      if (rc != PW_OK) break;
      GradArgs ma;
      std::memset(&ma, 0, sizeof(ma));
      ma.partial = m.partial;
      ma.n_split = m.n_split;
      ma.W = m.W;
      ma.D = m.D;
      GradOut o;
      std::memset(&o, 0, sizeof(o));
      o.own = side == 0 ? out->dX : out->dY;
      o.ld_own = side == 0 ? out->lddx : out->lddy;
      if (side == 1) {
        o.dV = out->dV;
        o.lddv = out->lddv;
      }
      rc = hip_status(launch_grad_merge(e->dtype, ma, side, side == 0 ? e->N : e->M,
                                        (side == 1 && cons == C_SOFTMAX) ? (int)C : 0, o, s));
      if (side == last_side && tile_ev_stop) (void)hipEventRecord(tile_ev_stop, s);
    }
    return rc;
  }
  for (int side = 0; side < 2 && rc == PW_OK; ++side) {
    if (!want_side(side)) continue;
    if (!started && tile_ev_start) (void)hipEventRecord(tile_ev_start, s);
    started = true;
    a.n_rb = g.n_rb[side];
    a.n_split = g.n_split[side];
    a.split = g.split[side];
    a.W = g.W[side];
    a.partial = base + g.off_part;
    rc = hip_status(grad_launch(e->dtype, e->metric, cons, side, g.dt, g.ct, a, s));
    if (rc != PW_OK) break;
    GradOut o;
    std::memset(&o, 0, sizeof(o));
    o.own = side == 0 ? out->dX : out->dY;
    o.ld_own = side == 0 ? out->lddx : out->lddy;
    if (side == 1) {
      o.dV = out->dV;
      o.lddv = out->lddv;
    }
    for (int t = 0; t < a.n_ops; ++t)
      if (a.ops[t].where == side + 1) o.dop[t] = out->dops[bound_of[t]];
    rc = hip_status(launch_grad_merge(e->dtype, a, side, side == 0 ? e->N : e->M, (side == 1 && value) ? (int)C : 0,
                                      o, s));
    if (side == last_side && tile_ev_stop) (void)hipEventRecord(tile_ev_stop, s);
  }
  return rc;
}

}  // extern "C"

// ------------------------------------------------------------------ CG solve

namespace {

// Workspace of a CG solve: the kernel product's own workspace, the iterates
// R, P, Q [N, C], the column partials and the per-column state.
struct CgLayout {
  size_t mm = 0, r = 0, p = 0, q = 0, part = 0, st = 0, total = 0;
};

CgLayout cg_layout(const pw_expr &e, int64_t C) {
  CgLayout L;
  const size_t es = esize(e.dtype);
  const Plan mp = make_plan(e, PW_C_MATMUL, C, 0);
  size_t off = align_up(mp.total);
  const size_t vec = align_up((size_t)e.N * (size_t)C * es);
  L.r = off;
  off += vec;
  L.p = off;
  off += vec;
  L.q = off;
  off += vec;
  L.part = off;
  off += align_up((size_t)cg_blocks(e.N) * (size_t)C * sizeof(double));
  L.st = off;
  off += align_up((size_t)C * (4 * sizeof(double) + sizeof(int)));
  L.total = off + kAlign;
  return L;
}

}  // namespace

extern "C" {

int pw_cg_workspace_size(const pw_expr *e, int64_t C, size_t *bytes) {
  if (!e || !bytes || C < 1) return PW_ERR_INVALID;
  if (e->B > 1) return PW_ERR_UNSUPPORTED;  // one system per solve
  *bytes = cg_layout(*e, C).total;
  return PW_OK;
}

int pw_cg_solve(const pw_expr *e, double shift, const void *B, int64_t C, int64_t ldb, void *A, int64_t lda,
                int max_iter, double rtol, int check_every, void *ws, size_t ws_bytes, void *stream,
                pw_solve_info *info) {
  if (!e || !info || e->N != e->M || C < 1 || ldb < C || lda < C) return PW_ERR_INVALID;
  if (e->B > 1) return PW_ERR_UNSUPPORTED;
  if (!(std::isfinite(shift) && shift > 0) || !(std::isfinite(rtol) && rtol >= 0)) return PW_ERR_INVALID;
  if (max_iter < 1 || check_every < 1) return PW_ERR_INVALID;
  const size_t es = esize(e->dtype);
  if (e->N > 0 && (!B || !A)) return PW_ERR_INVALID;
  if (!aligned(B, es) || !aligned(A, es)) return PW_ERR_INVALID;
  if (C > INT32_MAX) return PW_ERR_UNSUPPORTED;
  info->converged = 1;
  info->status = PW_SOLVE_CONVERGED;
  info->iterations = 0;
  info->max_rel_residual = 0.0;
  if (e->N == 0) return PW_OK;
  const CgLayout L = cg_layout(*e, C);
  if (!ws || ws_bytes < L.total) return PW_ERR_WORKSPACE;
  char *base = reinterpret_cast<char *>(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
  hipStream_t s = (hipStream_t)stream;
  const int nC = (int)C;
  void *R = base + L.r, *P = base + L.p, *Q = base + L.q;
  double *part = reinterpret_cast<double *>(base + L.part);
  CgState st;
  double *sd = reinterpret_cast<double *>(base + L.st);
  st.rr = sd;
  st.bb = sd + C;
  st.alpha = sd + 2 * C;
  st.beta = sd + 3 * C;
  st.flag = reinterpret_cast<int *>(sd + 4 * C);
  const int nblk = cg_blocks(e->N);
  const double tol2 = rtol * rtol;
  const size_t mm_bytes = L.r;  // the product's workspace sits first

  int rc = hip_status(launch_cg_init(e->dtype, B, ldb, A, lda, R, P, e->N, nC, part, s));
  if (rc == PW_OK) rc = hip_status(launch_cg_scalars(0, part, nblk, nC, st, tol2, s));
  std::vector<int> flag(C);
  auto running = [&](int *any_running, int *any_breakdown) -> int {
    int r = hip_status(hipMemcpyAsync(flag.data(), st.flag, C * sizeof(int), hipMemcpyDeviceToHost, s));
    if (r == PW_OK) r = hip_status(hipStreamSynchronize(s));
    *any_running = *any_breakdown = 0;
    for (int c = 0; c < nC; ++c) {
      *any_running |= flag[c] == 1;
      *any_breakdown |= flag[c] == 2;
    }
    return r;
  };
  int any_run = 1, any_brk = 0, it = 0;
  if (rc == PW_OK) rc = running(&any_run, &any_brk);
  while (rc == PW_OK && any_run && it < max_iter) {
    rc = value_consumer(e, PW_C_MATMUL, P, C, C, Q, C, base, mm_bytes, stream);
    if (rc == PW_OK) rc = hip_status(launch_cg_pq(e->dtype, P, Q, e->N, nC, shift, part, s));
    if (rc == PW_OK) rc = hip_status(launch_cg_scalars(1, part, nblk, nC, st, tol2, s));
    if (rc == PW_OK) rc = hip_status(launch_cg_update(e->dtype, P, Q, A, lda, R, e->N, nC, st, part, s));
    if (rc == PW_OK) rc = hip_status(launch_cg_scalars(2, part, nblk, nC, st, tol2, s));
    if (rc == PW_OK) rc = hip_status(launch_cg_direction(e->dtype, R, P, e->N, nC, st, s));
    ++it;
    if (rc == PW_OK && (it % check_every == 0 || it == max_iter)) rc = running(&any_run, &any_brk);
  }
  if (rc != PW_OK) return rc;
  std::vector<double> rr(C), bb(C);
  rc = hip_status(hipMemcpyAsync(rr.data(), st.rr, C * sizeof(double), hipMemcpyDeviceToHost, s));
  if (rc == PW_OK) rc = hip_status(hipMemcpyAsync(bb.data(), st.bb, C * sizeof(double), hipMemcpyDeviceToHost, s));
  if (rc == PW_OK) rc = hip_status(hipStreamSynchronize(s));
  if (rc != PW_OK) return rc;
  double worst = 0.0;
  for (int c = 0; c < nC; ++c)
    if (bb[c] > 0) worst = std::max(worst, std::sqrt(rr[c] / bb[c]));
  info->iterations = it;
  info->max_rel_residual = worst;
  info->status = any_brk ? PW_SOLVE_BREAKDOWN : (any_run ? PW_SOLVE_MAX_ITER : PW_SOLVE_CONVERGED);
  info->converged = info->status == PW_SOLVE_CONVERGED;
  return PW_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Squared MMD: three batched kernel products with a column of ones (within
// X, within Y, across). The unbiased statistic's within-cloud sums take the
// strict upper triangle (band mask: keep j >= i + 1) and count it twice; all
// built-in metrics are symmetric. One finishing kernel per batch element.
// ---------------------------------------------------------------------------
namespace {

struct MmdExprs {
  ExprHolder xx, yy, xy;
};

int mmd_bind(int dtype, int metric, double gamma, const void *X, int64_t n, int64_t ldx, int64_t sx, const void *Y,
             int64_t m, int64_t ldy, int64_t sy, int64_t D, int64_t B, bool unbiased, MmdExprs *ex) {
  pw_op upper{};
  upper.kind = PW_OP_BAND_LOWER;  // i - j <= -1
  upper.scalar = -1.0;
  const int n_ops = unbiased ? 1 : 0;
  pw_batch bx{}, by{}, bxy{};
  bx.B = by.B = bxy.B = B;
  bx.sx = bx.sy = sx;
  by.sx = by.sy = sy;
  bxy.sx = sx;
  bxy.sy = sy;
  int rc = bind_impl(&ex->xx.e, dtype, metric, gamma, X, n, ldx, X, n, ldx, D, &upper, n_ops, &bx);
  if (rc == PW_OK) rc = bind_impl(&ex->yy.e, dtype, metric, gamma, Y, m, ldy, Y, m, ldy, D, &upper, n_ops, &by);
  if (rc == PW_OK) rc = bind_impl(&ex->xy.e, dtype, metric, gamma, X, n, ldx, Y, m, ldy, D, nullptr, 0, &bxy);
  return rc;
}

// Workspace: ones [max(n, m)], row sums rxx [B][n], ryy [B][m], rxy [B][n],
// then the largest of the three products' workspaces.
struct MmdLayout {
  size_t rxx = 0, ryy = 0, rxy = 0, prod = 0, prod_bytes = 0, total = 0;
};

MmdLayout mmd_layout(const MmdExprs &ex) {
  MmdLayout L;
  const pw_expr &x = *ex.xx.e;
  const size_t es = esize(x.dtype), n = (size_t)x.N, m = (size_t)ex.yy.e->N, B = (size_t)x.B;
  size_t off = align_up(std::max(n, m) * es);
  L.rxx = off;
  off += align_up(B * n * es);
  L.ryy = off;
  off += align_up(B * m * es);
  L.rxy = off;
  off += align_up(B * n * es);
  L.prod = off;
  for (const pw_expr *e : {ex.xx.e, ex.yy.e, ex.xy.e})
    L.prod_bytes = std::max(L.prod_bytes, make_plan(*e, PW_C_MATMUL, 1, 0).total);
  L.total = off + L.prod_bytes + kAlign;
  return L;
}

int mmd_check_sizes(int64_t n, int64_t m, int64_t B, int unbiased) {
  if (unbiased != 0 && unbiased != 1) return PW_ERR_INVALID;
  if (B < 1 || n < (unbiased ? 2 : 1) || m < (unbiased ? 2 : 1)) return PW_ERR_INVALID;
  return PW_OK;
}

}  // namespace

extern "C" {

int pw_mmd2_workspace_size(int dtype, int metric, double gamma, int64_t n, int64_t m, int64_t D, int64_t B,
                           size_t *bytes) {
  if (!bytes) return PW_ERR_INVALID;
  *bytes = 0;
  int rc = mmd_check_sizes(n, m, B, 0);
  if (rc != PW_OK) return rc;
  // Sizes only: aligned stand-in pointers, and per-element clouds (the
  // larger workspace of the two stride cases).
  const void *fake = reinterpret_cast<const void *>(kAlign);
  MmdExprs ex;
  rc = mmd_bind(dtype, metric, gamma, fake, n, D, 1, fake, m, D, 1, D, B, true, &ex);
  if (rc != PW_OK) return rc;
  MmdExprs exb;
  rc = mmd_bind(dtype, metric, gamma, fake, n, D, 1, fake, m, D, 1, D, B, false, &exb);
  if (rc != PW_OK) return rc;
  *bytes = std::max(mmd_layout(ex).total, mmd_layout(exb).total);
  return PW_OK;
}

int pw_mmd2(int dtype, int metric, double gamma, const void *X, int64_t n, int64_t ldx, int64_t sx, const void *Y,
            int64_t m, int64_t ldy, int64_t sy, int64_t D, int64_t B, int unbiased, void *out, void *ws,
            size_t ws_bytes, void *stream) {
  int rc = mmd_check_sizes(n, m, B, unbiased);
  if (rc != PW_OK) return rc;
  if (dtype != PW_F32 && dtype != PW_F64) return PW_ERR_INVALID;
  if (!out || !aligned(out, esize(dtype))) return PW_ERR_INVALID;
  MmdExprs ex;
  rc = mmd_bind(dtype, metric, gamma, X, n, ldx, sx, Y, m, ldy, sy, D, B, unbiased != 0, &ex);
  if (rc != PW_OK) return rc;
  const MmdLayout L = mmd_layout(ex);
  if (!ws || ws_bytes < L.total) return PW_ERR_WORKSPACE;
  char *base = reinterpret_cast<char *>(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
  hipStream_t s = (hipStream_t)stream;
  void *ones = base, *rxx = base + L.rxx, *ryy = base + L.ryy, *rxy = base + L.rxy;
  rc = hip_status(launch_fill(dtype, ones, std::max(n, m), 1, 1, 1.0, s));
  if (rc == PW_OK) rc = value_consumer(ex.xx.e, PW_C_MATMUL, ones, 1, 1, rxx, 1, base + L.prod, L.prod_bytes, stream);
  if (rc == PW_OK) rc = value_consumer(ex.yy.e, PW_C_MATMUL, ones, 1, 1, ryy, 1, base + L.prod, L.prod_bytes, stream);
  if (rc == PW_OK) rc = value_consumer(ex.xy.e, PW_C_MATMUL, ones, 1, 1, rxy, 1, base + L.prod, L.prod_bytes, stream);
  if (rc != PW_OK) return rc;
  const double dn = (double)n, dm = (double)m;
  const double cx = unbiased ? 2.0 / (dn * (dn - 1.0)) : 1.0 / (dn * dn);
  const double cy = unbiased ? 2.0 / (dm * (dm - 1.0)) : 1.0 / (dm * dm);
  return hip_status(launch_mmd_finish(dtype, rxx, ryy, rxy, n, m, B, cx, cy, 2.0 / (dn * dm), out, s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// MMD backward: per batch element, pw_backward of the three products with
// ones (the unbiased within-cloud ones over the strict upper triangle, whose
// two sides are the two members of each distinct pair), then one combining
// kernel per cloud.
// ---------------------------------------------------------------------------
namespace {

// Workspace: ones [max(n, m)], six gradient blocks (within X: rows and
// columns [n][D]; within Y: [m][D] twice; across: X side [n][D], Y side
// [m][D]), then the largest pw_backward workspace of the three products.
struct MmdGradLayout {
  size_t t[6] = {0, 0, 0, 0, 0, 0}, bwd = 0, bwd_bytes = 0, total = 0;
};

MmdGradLayout mmd_grad_layout(const MmdExprs &ex) {
  MmdGradLayout L;
  const pw_expr &x = *ex.xx.e;
  const size_t es = esize(x.dtype), n = (size_t)x.N, m = (size_t)ex.yy.e->N, D = (size_t)x.D;
  size_t off = align_up(std::max(n, m) * es);
  const size_t rows[6] = {n, n, m, m, n, m};
  for (int q = 0; q < 6; ++q) {
    L.t[q] = off;
    off += align_up(rows[q] * D * es);
  }
  L.bwd = off;
  for (const pw_expr *e : {ex.xx.e, ex.yy.e, ex.xy.e})
    L.bwd_bytes = std::max(L.bwd_bytes, grad_plan(*e, PW_C_MATMUL, 1).total);
  L.total = off + L.bwd_bytes + kAlign;
  return L;
}

}  // namespace

extern "C" {

int pw_mmd2_backward_workspace_size(int dtype, int metric, double gamma, int64_t n, int64_t m, int64_t D,
                                    size_t *bytes) {
  if (!bytes) return PW_ERR_INVALID;
  *bytes = 0;
  int rc = mmd_check_sizes(n, m, 1, 0);
  if (rc != PW_OK) return rc;
  const void *fake = reinterpret_cast<const void *>(kAlign);
  size_t most = 0;
  for (bool unbiased : {true, false}) {
    MmdExprs ex;
    rc = mmd_bind(dtype, metric, gamma, fake, n, D, 0, fake, m, D, 0, D, 1, unbiased, &ex);
    if (rc != PW_OK) return rc;
    most = std::max(most, mmd_grad_layout(ex).total);
  }
  *bytes = most;
  return PW_OK;
}

int pw_mmd2_backward(int dtype, int metric, double gamma, const void *X, int64_t n, int64_t ldx, int64_t sx,
                     const void *Y, int64_t m, int64_t ldy, int64_t sy, int64_t D, int64_t B, int unbiased,
                     const void *G, void *dX, int64_t lddx, void *dY, int64_t lddy, void *ws, size_t ws_bytes,
                     void *stream) {
  int rc = mmd_check_sizes(n, m, B, unbiased);
  if (rc != PW_OK) return rc;
  if (dtype != PW_F32 && dtype != PW_F64) return PW_ERR_INVALID;
  const size_t es = esize(dtype);
  if (sx < 0 || sy < 0) return PW_ERR_INVALID;
  if (!G || !aligned(G, es)) return PW_ERR_INVALID;
  if ((dX && (lddx < D || !aligned(dX, es))) || (dY && (lddy < D || !aligned(dY, es)))) return PW_ERR_INVALID;
  // Validate every argument (and size the work) on element 0 before any
  // device work.
  MmdExprs ex0;
  rc = mmd_bind(dtype, metric, gamma, X, n, ldx, 0, Y, m, ldy, 0, D, 1, unbiased != 0, &ex0);
  if (rc != PW_OK) return rc;
  const MmdGradLayout L = mmd_grad_layout(ex0);
  if (!ws || ws_bytes < L.total) return PW_ERR_WORKSPACE;
  if (!dX && !dY) return PW_OK;
  char *base = reinterpret_cast<char *>(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
  hipStream_t s = (hipStream_t)stream;
  void *ones = base;
  void *t[6];
  for (int q = 0; q < 6; ++q) t[q] = base + L.t[q];
  rc = hip_status(launch_fill(dtype, ones, std::max(n, m), 1, 1, 1.0, s));
  const double dn = (double)n, dm = (double)m;
  const double cx = unbiased ? 2.0 / (dn * (dn - 1.0)) : 1.0 / (dn * dn);
  const double cy = unbiased ? 2.0 / (dm * (dm - 1.0)) : 1.0 / (dm * dm);
  const double cxy = 2.0 / (dn * dm);
  pw_grad_in in{};
  in.G = ones;
  in.ldg = 1;
  in.V = ones;
  in.C = 1;
  in.ldv = 1;
  for (int64_t b = 0; b < B && rc == PW_OK; ++b) {
    const char *Xb = static_cast<const char *>(X) + b * sx * (int64_t)es;
    const char *Yb = static_cast<const char *>(Y) + b * sy * (int64_t)es;
    MmdExprs ex;
    rc = mmd_bind(dtype, metric, gamma, Xb, n, ldx, 0, Yb, m, ldy, 0, D, 1, unbiased != 0, &ex);
    if (rc != PW_OK) break;
    pw_grad_out o{};
    if (dX) {
      o.dX = t[0];
      o.lddx = D;
      o.dY = t[1];
      o.lddy = D;
      rc = pw_backward(ex.xx.e, PW_C_MATMUL, &in, &o, base + L.bwd, L.bwd_bytes, stream);
    }
    if (rc == PW_OK && dY) {
      o.dX = t[2];
      o.lddx = D;
      o.dY = t[3];
      o.lddy = D;
      rc = pw_backward(ex.yy.e, PW_C_MATMUL, &in, &o, base + L.bwd, L.bwd_bytes, stream);
    }
    if (rc == PW_OK) {
      o.dX = dX ? t[4] : nullptr;
      o.lddx = D;
      o.dY = dY ? t[5] : nullptr;
      o.lddy = D;
      rc = pw_backward(ex.xy.e, PW_C_MATMUL, &in, &o, base + L.bwd, L.bwd_bytes, stream);
    }
    if (rc == PW_OK && dX) {
      const bool shared = sx == 0;
      char *out = static_cast<char *>(dX) + (shared ? 0 : b * n * lddx * (int64_t)es);
      rc = hip_status(launch_mmd_grad_combine(dtype, t[0], t[1], t[4], n, D, G, b, cx, cxy, out, lddx,
                                              shared && b > 0, s));
    }
    if (rc == PW_OK && dY) {
      const bool shared = sy == 0;
      char *out = static_cast<char *>(dY) + (shared ? 0 : b * m * lddy * (int64_t)es);
      rc = hip_status(launch_mmd_grad_combine(dtype, t[2], t[3], t[5], m, D, G, b, cy, cxy, out, lddy,
                                              shared && b > 0, s));
    }
  }
  return rc;
}

}  // extern "C"
