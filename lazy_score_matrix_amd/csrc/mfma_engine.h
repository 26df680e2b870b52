// Matrix-core (MFMA) tile engine for gfx950.
//
// Used when the feature dimension makes X.Y^T a real contraction (D >= 16).
// A workgroup of 4 waves owns BM query rows; every wave owns QB blocks of TM
// queries and streams the workgroup's column range through LDS tiles of 64
// keys. Per TM-key sub-block a wave computes the TRANSPOSED score block
// S^T = K . Q^T on the matrix cores:
//   float:  v_mfma_f32_32x32x2f32  (TM = 32; lane l holds query l%32 and the
//           16 keys 8*(r/4) + 4*(l/32) + r%4, r = 0..15)
//   double: v_mfma_f64_16x16x4f64  (TM = 16; lane l holds query l%16 and the
//           4 keys 4*r + l/16, r = 0..3)
// so each lane holds one query's scores and a row reduction needs only a
// register fold plus one or two cross-lane exchanges. The same registers are
// directly the B operand of the second contraction O^T += V^T . P (matmul,
// softmax@V, displacement), whose accumulator again keeps one query per lane.
//
// Distances use |x|^2 + |y|^2 - 2 x.y: the query operand is pre-scaled by -2
// (exact) and the accumulator starts at |x_i|^2 + |y_j|^2, so the matrix
// cores return the squared distance directly; it is clamped at 0. Cosine
// distance is 1 - (x.y) (1/|x_i|) (1/|y_j|) with the inverse norms from a
// pre-pass (columns) and from the query operand (rows).
//
// Epilogue: this engine takes chains that reduce to one affine stage with
// row terms only (s <- r_i s + p_i, scalars or per-row vectors); any other
// chain runs on the VALU engine. For logsumexp and softmax the scores are
// kept in base 2 (log2(e) folded into r_i), p_i is added once at the end
// for logsumexp and drops out of softmax.
#pragma once

#include "device_common.h"

namespace pw {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <class T>
struct Mfma;

template <>
struct Mfma<float> {
  static constexpr int TM = 32, G = 2, NREG = 16;
  typedef f32x16 acc_t;
  __device__ __forceinline__ static int key_of(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }
  __device__ __forceinline__ static acc_t mma(float a, float b, const acc_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // Lanes l and l^32 hold the same query: one cross-half lane swap leaves
  // {v[l], v[l^32]} in the two result registers of every lane.
  __device__ __forceinline__ static float gmax(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  __device__ __forceinline__ static float gsum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  __device__ __forceinline__ static float exp2(float x) { return __builtin_amdgcn_exp2f(x); }
  __device__ __forceinline__ static float log(float x) { return __builtin_amdgcn_logf(x) * kLn2_f; }
};

template <>
struct Mfma<double> {
  static constexpr int TM = 16, G = 4, NREG = 4;
  typedef f64x4 acc_t;
  __device__ __forceinline__ static int key_of(int r, int g) { return 4 * r + g; }
  __device__ __forceinline__ static acc_t mma(double a, double b, const acc_t &c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  // Lanes l, l^16, l^32, l^48 hold the same query: two lane swaps (16 and
  // 32 apart), each leaving {v[l], v[l^d]} in the two result registers.
  template <int D>
  __device__ __forceinline__ static void swap2(double v, double &a, double &b) {
    const uint32_t lo = (uint32_t)__double_as_longlong(v), hi = (uint32_t)(__double_as_longlong(v) >> 32);
    auto rl = D == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                      : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    auto rh = D == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                      : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    a = __longlong_as_double((long long)(((uint64_t)rh[0] << 32) | rl[0]));
    b = __longlong_as_double((long long)(((uint64_t)rh[1] << 32) | rl[1]));
  }
  __device__ __forceinline__ static double gmax(double v) {
    double a, b;
    swap2<16>(v, a, b);
    swap2<32>(fmax(a, b), a, b);
    return fmax(a, b);
  }
  __device__ __forceinline__ static double gsum(double v) {
    double a, b;
    swap2<16>(v, a, b);
    swap2<32>(a + b, a, b);
    return a + b;
  }
  __device__ __forceinline__ static double exp2(double x) { return ::exp2(x); }
  __device__ __forceinline__ static double log(double x) { return ::log(x); }
};

// Table-driven 2^x in double (Tang's method): with t = 256 x (exact),
// n = round(t) and f = t - n (exact, |f| <= 1/2),
//   2^x = 2^floor(n/256) * 2^((n mod 256)/256) * e^(a f),  a = ln2/256,
// where the middle factor comes from a 256-entry table in LDS and
// e^(a f) - 1 from its Taylor polynomial to degree 4 (|a f| <= 1.36e-3, so
// the first omitted term is below 4e-17). The scale by 2^floor(n/256) is an
// ldexp, which also flushes far-underflowing results to zero; t is clamped
// at -2^30 so that x = -inf gives 0.
__device__ __forceinline__ double exp2_table(double x, const double *__restrict__ tab, const double (&c)[4]) {
  const double t = fmax(x * 256.0, -1073741824.0);
  const double nd = rint(t);
  const double f = t - nd;
  const int n = (int)nd;
  const double p = f * fma(f, fma(f, fma(f, c[3], c[2]), c[1]), c[0]);
  const double T = tab[n & 255];
  return ldexp(fma(T, p, T), n >> 8);
}

__device__ __forceinline__ Key<float> key_placeholder(Key<float>) { return Key<float>{0ull}; }
__device__ __forceinline__ Key<double> key_placeholder(Key<double>) { return Key<double>{0ull, 0u}; }
// Cooperative loader of a [ROWS, COLS] tile (COLS padded, zero beyond the
// valid columns and rows) through registers: load() issues the global reads
// for the next tile before the current one is computed, store() writes them
// to LDS after it. A full, unpadded, 16-byte aligned tile takes the fast
// path: one vector read per slot from a uniform tile base plus a per-thread
// offset computed once. Other tiles read element by element with bounds.
template <class T, int ROWS, int COLS, int NT>
struct TileLoader {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int VPR = COLS / VEC;  // vectors per row
  static constexpr int NV = (ROWS * VPR + NT - 1) / NT;
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  // Slot v of a thread is row tid / VPR + v * (NT / VPR), column
  // (tid % VPR) * VEC: one offset per thread and a uniform step, so the
  // slots need no address register each.
  static_assert(NT % VPR == 0, "a thread's slots are whole rows apart");
  static constexpr int RSTEP = NT / VPR;
  vec_t buf[NV];
  uint32_t off0;  // element offset of the thread's first slot inside a full tile
  bool fast;      // offsets fit 32 bits and rows are vector aligned

  __device__ __forceinline__ void init(int64_t ld, bool vec_ok, int tid) {
    fast = vec_ok && (int64_t)ROWS * ld < (int64_t)1 << 31;
    off0 = (uint32_t)((tid / VPR) * ld + (tid % VPR) * VEC);
  }
  __device__ __forceinline__ void load(const T *__restrict__ src, int64_t ld, int64_t row0, int nrows, int ncols,
                                       int tid) {
    if (fast && nrows == ROWS && ncols == COLS) {
      const T *__restrict__ base = src + row0 * ld + off0;
      const uint32_t step = (uint32_t)(RSTEP * ld);
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (ROWS * VPR % NT == 0 || tid + v * NT < ROWS * VPR)
          buf[v] = *reinterpret_cast<const vec_t *>(base + v * step);
      return;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * NT;
      const int r = idx / VPR, c = (idx % VPR) * VEC;
      vec_t x;
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        x[e] = (idx < ROWS * VPR && r < nrows && c + e < ncols) ? src[(row0 + r) * ld + c + e] : (T)0;
      buf[v] = x;
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(T (*dst)[LD], int tid) const {
    T *p = &dst[tid / VPR][(tid % VPR) * VEC];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (ROWS * VPR % NT == 0 || tid + v * NT < ROWS * VPR)
        *reinterpret_cast<vec_t *>(p + v * RSTEP * LD) = buf[v];
    }
  }
};

__device__ __forceinline__ bool vec_ok(const void *p, int64_t ld, int vec) {
  return ((uintptr_t)p % 16 == 0) && (ld % vec == 0);
}

template <class T, int CONS, int DP, int CP, int KL>
struct MfmaShape {
  static constexpr int DT = sizeof(T) == 4 ? 0 : 1;
  static constexpr int WAVES = mfma_waves(DT, DP, CP, KL);
  static constexpr int NT = WAVES * 64;
  static constexpr int QB = (sizeof(T) == 8 && CONS != C_TOPK) ? 2 : 1;
  static constexpr int BM = WAVES * QB * Mfma<T>::TM;
  static_assert(BM == mfma_bm(DT, CONS, DP, CP, KL), "host and device row-block sizes differ");
};

// MASKED instantiations carry the mask logic (row flags, per-key flags and
// group ids in LDS, tile classes, keep bits); the others compile without it
// and keep their register budget.
template <class T, int METRIC, int CONS, int DP, int CP, int KL, bool MASKED>
__global__ __launch_bounds__((MfmaShape<T, CONS, DP, CP, KL>::NT),
                             (mfma_wgs_per_cu(sizeof(T) == 4 ? 0 : 1, CONS, DP, CP, KL))) void mfma_tile(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  using F = Mfma<T>;
  using acc_t = typename F::acc_t;
  constexpr int TM = F::TM, G = F::G, NREG = F::NREG;
  using Shape = MfmaShape<T, CONS, DP, CP, KL>;
  constexpr int QB = Shape::QB;
  constexpr int BM = Shape::BM;
  constexpr int NT = Shape::NT;
  constexpr int BN = mfma_bn(sizeof(T) == 4 ? 0 : 1, CONS, CP, DP);
  constexpr int SB = BN / TM;
  constexpr int DG = DP / G;
  constexpr bool DIST = METRIC == M_SQEUCLIDEAN || METRIC == M_RBF;  // norm expansion
  constexpr bool COS = METRIC == M_COSINE;
  constexpr bool NEEDN = DIST || COS;  // a per-key norm term staged in sN
  constexpr bool HAS_V = CONS == C_MATMUL || CONS == C_SOFTMAX;
  // A single value column (a weighted row sum): V is staged as one LDS
  // column and folded with vector FMAs; the matrix cores compute the scores.
  constexpr bool NARROW = CONS == C_MATMUL && CP == 1;
  constexpr bool VTILE = HAS_V && !NARROW;
  constexpr bool ONLINE = CONS == C_LOGSUMEXP || CONS == C_SOFTMAX;
  constexpr int NCB = VTILE ? CP / TM : (CONS == C_DISPLACEMENT ? (DP + TM - 1) / TM : 1);
  constexpr bool PV = VTILE || CONS == C_DISPLACEMENT;
  static_assert(BN <= NT, "one thread stages each key's norm and value");
  constexpr int KPAD = sizeof(T) == 4 ? 4 : 2;
  constexpr int VW = HAS_V ? CP : 1;
  constexpr int KLQ = CONS == C_TOPK ? KL : 1;
  constexpr T kNegInf = -__builtin_huge_valf();

  // Two LDS buffers per tile array: tile t+1 is written into one while
  // tile t is read from the other, so each tile costs a single barrier.
  __shared__ __attribute__((aligned(16))) T sKb[2][BN][DP + KPAD];
  __shared__ __attribute__((aligned(16))) T sNb[2][BN];
  __shared__ __attribute__((aligned(16))) T sVb[2][HAS_V ? BN : 1][VW];
  constexpr int MBN = MASKED ? BN : 1;
  __shared__ int sCb[2][MBN];      // column mask flags
  __shared__ int64_t sGb[2][MBN];  // column group ids
  T(*sK)[DP + KPAD] = sKb[0];
  T *sN = sNb[0];
  T(*sV)[VW] = sVb[0];
  int *sC = sCb[0];
  int64_t *sG = sGb[0];
  constexpr bool TABLE_EXP = sizeof(T) == 8 && (ONLINE || METRIC == M_RBF);
  __shared__ double sE[TABLE_EXP ? 256 : 1];

  const int tid = threadIdx.x;
  // 2^x: the hardware exponential for float, the LDS table for double (the
  // table is complete after the first barrier of the main loop).
  double ec[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) ec[k] = a.exp2_c[k];
  if constexpr (TABLE_EXP) {
    for (int j = tid; j < 256; j += NT) sE[j] = ::exp2((double)j / 256.0);
  }
  auto ex2 = [&](T x) -> T {
    if constexpr (TABLE_EXP) return exp2_table(x, sE, ec);
    else return F::exp2(x);
  };
  const int w = tid >> 6, l = tid & 63, g = l / TM, q = l % TM;
  // Row blocks of this workgroup: one, or with rb_pairs (masked launches
  // with a band) the pair r, n_rb - 1 - r, so the light rows at one end of
  // a causal band and the heavy rows at the other share a workgroup.
  const int rb_slots = (MASKED && a.rb_pairs) ? a.rb_pairs : a.n_rb;
  // Block coordinates are wave-uniform: keeping them (and the column range
  // below) in scalar registers keeps the tile loop's control scalar.
  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
  // Renumbering them XCD-major gives each XCD a contiguous run of blocks,
  // so the row blocks sharing a column split (and its key tiles) share an
  // L2.
  const int nblk = gridDim.x;
  const int bid = (nblk % 8 == 0) ? (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8 : blockIdx.x;
  const int slot = __builtin_amdgcn_readfirstlane(bid % rb_slots);
  const int sp = __builtin_amdgcn_readfirstlane(bid / rb_slots);
  const bool paired = MASKED && a.rb_pairs;
  // The slot's row blocks: by index, or by the pair order (heaviest with
  // lightest) when the launch has one.
  const int rb_first = (paired && a.rb_order) ? __builtin_amdgcn_readfirstlane(a.rb_order[slot]) : slot;
  const int rb_second = paired ? ((a.rb_order) ? __builtin_amdgcn_readfirstlane(a.rb_order[a.n_rb - 1 - slot])
                                               : a.n_rb - 1 - slot)
                               : slot;
  const int npass = (paired && rb_second != rb_first) ? 2 : 1;
  // Paired launches deal the pair's tiles (those of the first row block,
  // then those of the second, each within its band reach) out to the
  // splits in equal runs, so every workgroup gets the same number of tiles.
  int64_t pf[2] = {0, 0}, pl[2] = {0, 0}, pt[2] = {0, 0}, v0 = 0, v1 = 0;
  if (paired) {
    for (int p = 0; p < npass; ++p) {
      const int64_t q0 = (int64_t)(p ? rb_second : rb_first) * BM;
      band_range(a.mask, p ? rb_second : rb_first, q0, min(a.N, q0 + BM) - 1, 0, a.M, BN, &pf[p], &pl[p]);
      pt[p] = pl[p] > pf[p] ? (pl[p] - pf[p] + BN - 1) / BN : 0;
    }
    const int64_t tt = pt[0] + pt[1];
    v0 = tt * sp / a.n_split;
    v1 = tt * (sp + 1) / a.n_split;
  }
  for (int pass = 0; pass < npass; ++pass) {
  if (pass) __syncthreads();  // the previous row block's last LDS reads
  const int rb = pass ? rb_second : rb_first;
  const int64_t row0 = (int64_t)rb * BM;
  const int64_t jb = paired ? 0 : (int64_t)sp * a.split_cols;
  const int64_t je = wave_uniform(paired ? a.M : min(a.M, jb + a.split_cols));
  const T *__restrict__ Xp = static_cast<const T *>(bp.X);
  const T *__restrict__ Yp = static_cast<const T *>(bp.Y);
  const MaskArgs &mk = a.mask;
  const bool keyflags = MASKED && (mk.col || mk.grow);  // per-key mask data is staged
  const int64_t r1 = min(a.N, row0 + BM) - 1;

  // A paired pass whose run of tiles is empty reads no row operands; its
  // partial is the empty one.
  bool empty = false;
  if (paired) {
    const int64_t off = pass ? pt[0] : 0;
    empty = min(v1 - off, pt[pass]) <= max(v0 - off, (int64_t)0);
  }
  // ------------------------------------------------------------ row state
  int64_t qi[QB];
  bool qv[QB];
  T qr[QB][DG];
  T nx[QB];
  T er[QB], ep[QB];  // row epilogue: s <- er * s + ep
  bool rkeep[QB];    // row survives the row mask
  int64_t gq[QB];    // row group id
  const bool has_epi = a.epi.n_stages == 1;
  // A single-column product under a pure row scale (s <- r s, as a mean
  // binds it) scales the finished sum instead of every score.
  const bool epi_post = NARROW && has_epi && !a.epi.st[0].row_vec && a.epi.st[0].p_scalar == 0.0;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    qi[b] = row0 + (int64_t)(w * QB + b) * TM + q;
    qv[b] = qi[b] < a.N;
    rkeep[b] = qv[b] && (!MASKED || !mk.row || mk.row[qi[b]]);
    gq[b] = (MASKED && qv[b] && mk.grow) ? mk.grow[qi[b]] : 0;
    T part = 0;
#pragma unroll
    for (int s = 0; s < DG; ++s) {
      const int d = g * DG + s;
      T v = (qv[b] && !empty && d < a.D) ? Xp[qi[b] * a.ldx + d] : (T)0;
      part = fma(v, v, part);
      qr[b][s] = DIST ? (T)-2 * v : v;
    }
    nx[b] = F::gsum(part);
    if constexpr (COS) nx[b] = nx[b] > (T)0 ? (T)1 / sqrt(nx[b]) : (T)0;  // cosine keeps 1/|x_i| here
    T r = (T)1, p = (T)0;
    if (has_epi) {
      const Stage &st = a.epi.st[0];
      if (st.row_vec) {
        if (qv[b]) {
          r = ldg<T>(epi_vec(a, st.r_vec), qi[b]);
          p = ldg<T>(epi_vec(a, st.p_vec), qi[b]);
        }
      } else {
        r = (T)st.r_scalar;
        p = (T)st.p_scalar;
      }
    }
    if constexpr (ONLINE) r *= (T)kLog2e;  // base-2 scores
    er[b] = r;
    ep[b] = p;
    // Online consumers of a dot product: fold the row scale into the query
    // operand, so the matrix cores return the base-2 score directly.
    if constexpr (ONLINE && METRIC == M_LINEAR) {
#pragma unroll
      for (int s = 0; s < DG; ++s) qr[b][s] *= r;
      er[b] = (T)1;
    }
  }
  const T ngl2 = (T)(-a.gamma * kLog2e);
  // rbf: the accumulator holds u = |y_j|^2 - 2 x_i.y_j and the exponent is
  // u * c + |x_i|^2 * c, one FMA (c = -gamma log2(e), times 256 for the
  // double table, whose argument is 256 x).
  const T rbf_c = TABLE_EXP ? ngl2 * (T)256 : ngl2;
  T rbf_t[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) rbf_t[b] = rbf_c * nx[b];

  acc_t o[QB][NCB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int r = 0; r < NREG; ++r) o[b][c][r] = 0;
  T m[QB], lsum[QB], mass[QB];
  T wsum[QB][4];  // NARROW: four partial sums per row
  Key<T> list[QB][KLQ];
  T thr[QB];
  // Float top-k queues each lane's candidates (keys below the threshold as
  // it stood when they were met) in LDS and inserts them wave-wide later, so
  // one insertion serves every lane that has a candidate rather than one
  // lane at a time. Queues are per lane and in column order, and a queued
  // key enters only if still below the list's last value, so the result is
  // the same as inserting at once. The capacity is what the LDS left at this
  // kernel's occupancy allows; without room for a sub-block's candidates
  // and four more the kernel inserts at once.
  constexpr int kLdsPerCu = 160 * 1024;
  constexpr int LDS_USED = (int)sizeof(T) * (2 * BN * (DP + KPAD) + 2 * BN + 2 * (HAS_V ? BN : 1) * VW) +
                           (4 + 8) * 2 * MBN + (TABLE_EXP ? 2048 : 8) + 4 * (MASKED ? SB * QB * NT : 1);
  constexpr int QROOM = (kLdsPerCu / mfma_wgs_per_cu(sizeof(T) == 4 ? 0 : 1, CONS, DP, CP, KL) - LDS_USED - 1024) /
                        (NT * 8);
  constexpr int QCAP = QROOM < 32 ? QROOM : 32;
  constexpr bool QUEUE = CONS == C_TOPK && sizeof(T) == 4 && QB == 1 && QCAP >= NREG + 4;
  __shared__ uint64_t sQ[QUEUE ? QCAP : 1][QUEUE ? NT : 1];
  int qn = 0;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    thr[b] = __builtin_huge_valf();
    m[b] = kNegInf;
    lsum[b] = 0;
    mass[b] = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) wsum[b][u] = 0;
#pragma unroll
    for (int p = 0; p < KLQ; ++p)
      list[b][p] = (p < KLQ - a.k) ? key_placeholder(Key<T>()) : Key<T>::sentinel();
  }

  // ----------------------------------------------------------- sub-blocks
  // S^T for the TM keys at offset kb of the staged tile, all QB query blocks.
  // A plain search (PL) leaves |x_i|^2 out of the accumulator: it is the
  // same for every key of the row, so it is added once to the sub-block's
  // minimum and to each candidate instead of to every score.
  auto qk = [&](int kb, acc_t (&s)[QB], auto pl) __attribute__((always_inline)) {
    constexpr bool PL = decltype(pl)::value;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int r = 0; r < NREG; ++r)
        s[b][r] = DIST ? ((PL || METRIC == M_RBF) ? sN[kb + F::key_of(r, g)] : nx[b] + sN[kb + F::key_of(r, g)])
                       : (T)0;
    if constexpr (DG <= 16) {
      // A short operand run (at most 16 values) is read whole before the
      // first MFMA (the scheduling barrier keeps the compiler from sinking
      // the reads again), so its LDS latency is paid once per sub-block
      // rather than once per vector read.
      T av[DG];
#pragma unroll
      for (int st = 0; st < DG; ++st) av[st] = sK[kb + q][g * DG + st];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < DG; ++st) {
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b] = F::mma(av[st], qr[b][st], s[b]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < DG; ++st) {
        const T av = sK[kb + q][g * DG + st];
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b] = F::mma(av, qr[b][st], s[b]);
      }
    }
  };

  // Fold one sub-block of scores into the row reductions.
  // Keep bits of a checked sub-block: bit r of km[b] tells whether the pair
  // of query block b and register r survives the masks.
  auto keep_bits = [&](int kb, int64_t j0, uint32_t (&km)[QB]) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int64_t dbase = j0 + kb - qi[b];
      uint32_t bits = 0;
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        const int key = kb + F::key_of(r, g);
        bool kp = (!mk.col || sC[key]) && (!mk.grow || sG[key] == gq[b]);
        const int64_t d = dbase + F::key_of(r, g);
        kp = kp && (!mk.band || (d >= mk.lo && d <= mk.hi));
        bits |= (uint32_t)kp << r;
      }
      km[b] = bits;
    }
  };
  // Keep bits of every sub-block of a checked tile, formed once when the
  // tile starts (few registers are live there) and read back per sub-block.
  __shared__ uint32_t sKm[MASKED ? SB : 1][QB][MASKED ? NT : 1];
  // rbf kernel values of a sub-block. The exponent of a pair with x = y
  // can round slightly above 0, giving a value above 1 by a rounding error
  // of the distance; it is not clamped. For double the table lookups of all
  // registers are issued together, then used.
  auto rbf_values = [&](const acc_t (&s)[QB], T (&v)[QB][NREG]) __attribute__((always_inline)) {
    if constexpr (TABLE_EXP) {
      double p[QB][NREG];
      int n[QB][NREG];
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const double t = fmax(fma(s[b][r], rbf_c, rbf_t[b]), -1073741824.0);
          const double nd = rint(t);
          const double f = t - nd;
          n[b][r] = (int)nd;
          p[b][r] = f * fma(f, fma(f, fma(f, ec[3], ec[2]), ec[1]), ec[0]);
        }
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < NREG; ++r) v[b][r] = sE[n[b][r] & 255];
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < NREG; ++r) v[b][r] = ldexp(fma(v[b][r], p[b][r], v[b][r]), n[b][r] >> 8);
    } else {
      // The expansion can round a distance below zero (x = y) or, far from
      // the origin, well below it: the value is clamped to [0, 1], so k <= 1
      // (an overflow to +inf clamps to 1 as well). The clamp is the exp
      // instruction's own output clamp, which the median of (k, 0, 1)
      // compiles to: no instruction of its own. float64's rounding is 2^-52
      // of |x|^2: no clamp.
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < NREG; ++r)
          v[b][r] = __builtin_amdgcn_fmed3f(F::exp2(fma(s[b][r], rbf_c, rbf_t[b])), 0.f, 1.f);
    }
  };
  // Insert every lane's queued candidates, oldest first; the trip count is
  // the longest queue of the wave. Each entry is read from LDS one step
  // ahead, so the read's latency overlaps the previous insertion.
  auto drain = [&]() __attribute__((always_inline)) {
    if constexpr (QUEUE) {
      uint64_t nk = sQ[0][tid];
      for (int t = 0; __any(t < qn); ++t) {
        const Key<T> c{nk};
        if (t + 1 < QCAP) nk = sQ[t + 1][tid];
        if (t < qn) {
          if ((uint32_t)(c.k >> 32) < (uint32_t)(list[0][KLQ - 1].k >> 32)) {
            key_insert_after<KLQ>(list[0], c);
            thr[0] = key_threshold(list[0][KLQ - 1]);
          }
        }
      }
      qn = 0;
    }
  };
  auto consume = [&](int kb, int nb, int64_t j0, bool diag, bool check_, acc_t (&s)[QB], auto pl) __attribute__((always_inline)) {
    constexpr bool PL = decltype(pl)::value;
    const bool check = MASKED && check_;
    const bool tail = kb + TM > nb;
    uint32_t km[QB];
    if (check) {
#pragma unroll
      for (int b = 0; b < QB; ++b) km[b] = sKm[MASKED ? kb / TM : 0][b][MASKED ? tid : 0];
    }
    if constexpr (CONS == C_TOPK) {
      // Filter a whole sub-block with one wave vote before any insertion.
      // A plain search (no epilogue, smallest first, dot product or squared
      // distance) filters on the raw accumulator: its minimum plus |x_i|^2
      // (fl(n + u) is monotone in u, so this is the minimum of the sums) and
      // the clamp at 0 are applied to candidates only, as max(d, 0) < thr
      // implies d < thr.
      bool any = false;
      if constexpr (PL) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          if (check) {
#pragma unroll
            for (int r = 0; r < NREG; ++r)
              if (!((km[b] >> r) & 1u)) s[b][r] = __builtin_huge_valf();
          }
          T mn = s[b][0];
#pragma unroll
          for (int r = 1; r < NREG; ++r) mn = min(mn, s[b][r]);
          if constexpr (DIST) mn = nx[b] + mn;
          any |= mn < thr[b];
        }
      } else {
        T rv[QB][NREG];
        if constexpr (METRIC == M_RBF) rbf_values(s, rv);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          T mn = __builtin_huge_valf();
#pragma unroll
          for (int r = 0; r < NREG; ++r) {
            T x = s[b][r];
            if constexpr (METRIC == M_RBF) x = rv[b][r];
            else if constexpr (DIST) x = max(x, (T)0);
            if constexpr (COS) x = fma(-x * sN[kb + F::key_of(r, g)], nx[b], (T)1);
            x = fma(x, er[b], ep[b]);
            if (check && !((km[b] >> r) & 1u)) x = a.largest ? -__builtin_huge_valf() : __builtin_huge_valf();
            s[b][r] = x;
            mn = min(mn, a.largest ? -x : x);
          }
          any |= mn < thr[b];
        }
      }
      if (__any(any)) {
        if constexpr (QUEUE) {
          // A lane with a candidate may queue up to NREG keys: make room.
          if (__any(any && qn > QCAP - NREG)) drain();
          // A plain search compares n + u before the clamp at 0 (a clamped
          // value below the threshold implies it); the queued key carries
          // the clamped value, and the drain compares that. Only a ragged
          // sub-block checks the column range.
          auto push = [&](auto ragged) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NREG; ++r) {
              const int key = kb + F::key_of(r, g);
              T x = s[0][r];
              if (DIST && PL) x = nx[0] + x;
              const T sv = (!PL && a.largest) ? -x : x;
              if ((!decltype(ragged)::value || key < nb) && sv < thr[0]) {
                if (DIST && PL) x = max(x, (T)0);
                sQ[qn][tid] = Key<T>::make(x, (uint32_t)(j0 + key), PL ? 0 : a.largest).k;
                ++qn;
              }
            }
          };
          if (tail) push(Bool<true>());
          else push(Bool<false>());
        } else {
#pragma unroll
          for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int r = 0; r < NREG; ++r) {
              const int key = kb + F::key_of(r, g);
              T x = s[b][r];
              if (DIST && PL) x = max(nx[b] + x, (T)0);
              const T sv = (!PL && a.largest) ? -x : x;
              if (key < nb && sv < thr[b]) {
                key_insert_after<KLQ>(list[b], Key<T>::make(x, (uint32_t)(j0 + key), PL ? 0 : a.largest));
                thr[b] = key_threshold(list[b][KLQ - 1]);
              }
            }
        }
      }
      return;
    }

    // Finished score per register (base 2 for the online consumers).
    T v[QB][NREG];
    if constexpr (METRIC == M_RBF) rbf_values(s, v);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int r = 0; r < NREG; ++r) {
        T x = s[b][r];
        if constexpr (METRIC == M_RBF) x = v[b][r];
        else if constexpr (DIST) x = max(x, (T)0);
        if constexpr (COS) x = fma(-x * sN[kb + F::key_of(r, g)], nx[b], (T)1);
        if constexpr (ONLINE && METRIC != M_LINEAR) x = x * er[b];
        v[b][r] = x;
      }
      if constexpr (!ONLINE) {
        if (has_epi && !epi_post) {
#pragma unroll
          for (int r = 0; r < NREG; ++r) v[b][r] = fma(v[b][r], er[b], ep[b]);
        }
      }
      // The masks below apply to a few sub-blocks only (ragged, diagonal,
      // checked): marked unlikely, so they stay behind uniform branches
      // rather than becoming a select on every register of every sub-block.
      if (__builtin_expect(tail, 0)) {
#pragma unroll
        for (int r = 0; r < NREG; ++r)
          if (kb + F::key_of(r, g) >= nb) v[b][r] = ONLINE ? kNegInf : (T)0;
      }
      if (__builtin_expect(CONS == C_LOGSUMEXP && diag, 0)) {
#pragma unroll
        for (int r = 0; r < NREG; ++r)
          if (j0 + kb + F::key_of(r, g) == qi[b]) v[b][r] = kNegInf;
      }
      if (__builtin_expect(check, 0)) {
#pragma unroll
        for (int r = 0; r < NREG; ++r)
          if (!((km[b] >> r) & 1u)) v[b][r] = ONLINE ? kNegInf : (T)0;
      }
    }

    if constexpr (ONLINE) {
      // Online max/sum in base 2 with a lazily moved reference m: it only
      // moves when a block's maximum exceeds it by more than 8, so every
      // weight 2^(v - m) stays <= 256 and most blocks skip the rescale of
      // the running sums. The result divides by the sum taken with the same
      // reference, so the reference's value never enters it.
      bool need_any = false;
      T bmax[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        T bm = v[b][0];
#pragma unroll
        for (int r = 1; r < NREG; ++r) bm = max(bm, v[b][r]);
        bmax[b] = F::gmax(bm);
        need_any |= bmax[b] > m[b] + (T)8;
      }
      if (__any(need_any)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const bool need = bmax[b] > m[b] + (T)8;
          const T alpha = need ? ex2(m[b] - bmax[b]) : (T)1;
          m[b] = need ? bmax[b] : m[b];
          lsum[b] *= alpha;
          if constexpr (CONS == C_SOFTMAX) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) o[b][c] *= alpha;
          }
        }
      }
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const T mu = m[b] == kNegInf ? (T)0 : m[b];  // no valid key yet: weights are 2^-inf = 0
        T acc = 0;
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const T p = ex2(v[b][r] - mu);
          v[b][r] = p;
          acc += p;
        }
        lsum[b] += acc;
      }
    }

    if constexpr (NARROW) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < NREG; ++r) wsum[b][r % 4] = fma(v[b][r], sV[kb + F::key_of(r, g)][0], wsum[b][r % 4]);
    }

    if constexpr (PV) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
#pragma unroll
        for (int r = 0; r < NREG; ++r) {
          const int key = kb + F::key_of(r, g);
          T av;
          if constexpr (HAS_V) {
            av = sV[key][c * TM + q];
          } else {
            const int ch = c * TM + q;
            av = ch < DP ? sK[key][ch] : (T)0;
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) o[b][c] = F::mma(av, v[b][r], o[b][c]);
        }
      }
      if constexpr (CONS == C_DISPLACEMENT) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
          for (int r = 0; r < NREG; ++r) mass[b] += v[b][r];
      }
    }
  };

  // ------------------------------------------------------------ main loop
  // Register-prefetched tiles: the global reads of tile t+1 are in flight
  // while tile t is computed from LDS. Within a tile the scores of
  // sub-block sb+1 are issued to the matrix cores before sub-block sb is
  // consumed, so its vector work overlaps them.
  TileLoader<T, BN, DP, NT> ldK;
  TileLoader<T, BN, VTILE ? CP : 16 / (int)sizeof(T), NT> ldV;
  T nyv = 0, vcol = 0;
  int ckv = 0;
  int64_t gkv = 0;
  const bool kvec = vec_ok(bp.Y, a.ldy, 16 / (int)sizeof(T));
  const bool vvec = VTILE && vec_ok(bp.V, a.ldv, 16 / (int)sizeof(T));
  ldK.init(a.ldy, kvec, tid);
  if constexpr (VTILE) ldV.init(a.ldv, vvec, tid);
  auto prefetch = [&](int64_t t0) {
    const int nbt = (int)min((int64_t)BN, je - t0);
    ldK.load(Yp, a.ldy, t0, nbt, a.D, tid);
    if constexpr (VTILE) ldV.load(static_cast<const T *>(bp.V), a.ldv, t0, nbt, a.C, tid);
    if constexpr (NARROW) vcol = (tid < nbt) ? ldg<T>(bp.V, (t0 + tid) * a.ldv) : (T)0;
    if constexpr (NEEDN) nyv = (tid < nbt) ? ldg<T>(bp.ny, t0 + tid) : (T)0;
    if (keyflags) {
      ckv = (tid < nbt && (!mk.col || mk.col[t0 + tid])) ? 1 : 0;
      gkv = (tid < nbt && mk.grow) ? mk.gcol[t0 + tid] : 0;
    }
  };
  auto stage = [&](int buf) {
    ldK.store(sKb[buf], tid);
    if constexpr (VTILE) ldV.store(sVb[buf], tid);
    if constexpr (NARROW) {
      if (tid < BN) sVb[buf][tid][0] = vcol;
    }
    if constexpr (NEEDN) {
      if (tid < BN) sNb[buf][tid] = nyv;
    }
    if (keyflags && tid < BN) {
      sCb[buf][tid] = ckv;
      sGb[buf][tid] = gkv;
    }
  };
  // Tiles this row block visits: the band's reach inside the split, minus
  // tiles the masks drop whole.
  int64_t jfirst = jb, jlast = je;
  if constexpr (MASKED) {
    if (paired) {
      const int64_t off = pass ? pt[0] : 0;
      const int64_t t0 = max(v0 - off, (int64_t)0), t1 = min(v1 - off, pt[pass]);
      jfirst = pf[pass] + t0 * BN;
      jlast = t1 > t0 ? min(pl[pass], pf[pass] + t1 * BN) : jfirst;
    } else {
      band_range(mk, rb, row0, r1, jb, je, BN, &jfirst, &jlast);
    }
  }
  jfirst = wave_uniform(jfirst);
  jlast = wave_uniform(jlast);
  auto tile_cls = [&](int64_t t0) -> int {
    if constexpr (MASKED) return tile_class(mk, row0, r1, t0, min(t0 + BN, je) - 1, rb, t0 / BN);
    return TILE_FULL;
  };
  auto next_tile = [&](int64_t t0) {
    if constexpr (MASKED) {
      while (t0 < jlast && tile_cls(t0) == TILE_SKIP) t0 += BN;
    }
    return t0;
  };
  constexpr bool PLAIN_OK = CONS == C_TOPK && (METRIC == M_LINEAR || METRIC == M_SQEUCLIDEAN);
  const bool plain = PLAIN_OK && !has_epi && !a.largest;
  int buf = 0;
  int64_t j0 = next_tile(jfirst);
  if (j0 < jlast) {
    prefetch(j0);
    stage(0);
  }
  __syncthreads();

  // Plain searches (see consume) get a tile loop of their own, so their
  // list registers flow through a single loop.
  auto tile_loop = [&](auto pl) __attribute__((always_inline)) {
    while (j0 < jlast) {
      const int nb = (int)min((int64_t)BN, je - j0);
      const int64_t jn = next_tile(j0 + BN);
      const bool next = jn < jlast;
      if (next) prefetch(jn);
      sK = sKb[buf];
      sN = sNb[buf];
      sV = sVb[buf];
      sC = sCb[buf];
      sG = sGb[buf];
      const bool diag = CONS == C_LOGSUMEXP && a.exclude_self && j0 < row0 + BM && j0 + BN > row0;
      const bool check = tile_cls(j0) == TILE_CHECK;

      if (MASKED && check) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          uint32_t km[QB];
          keep_bits(sb * TM, j0, km);
#pragma unroll
          for (int b = 0; b < QB; ++b) sKm[MASKED ? sb : 0][b][MASKED ? tid : 0] = km[b];
        }
      }
      acc_t s0[QB], s1[QB];
      qk(0, s0, pl);
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        if (sb * TM >= nb) break;
        // Top-k issues the next sub-block's scores even past the tile's last
        // key (a ragged tile; the extra scores are never consumed): with no
        // branch around the issue, the compiler places the filter of this
        // sub-block between the next one's matrix instructions without a
        // long wait (k-NN 37.2 -> 36.6 ms; the other consumers measured
        // no better that way).
        const bool more = sb + 1 < SB && (CONS == C_TOPK || (sb + 1) * TM < nb);
        if (sb & 1) {
          if (more) qk((sb + 1) * TM, s0, pl);
          consume(sb * TM, nb, j0, diag, check, s1, pl);
        } else {
          if (more) qk((sb + 1) * TM, s1, pl);
          consume(sb * TM, nb, j0, diag, check, s0, pl);
        }
      }
      if (next) stage(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      j0 = jn;
    }
  };
  if constexpr (PLAIN_OK) {
    if (plain) tile_loop(Bool<true>());
    else tile_loop(Bool<false>());
  } else {
    tile_loop(Bool<false>());
  }
  drain();

  // Rows dropped by the row mask take the empty-row result.
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    if (MASKED && !rkeep[b]) {
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int r = 0; r < NREG; ++r) o[b][c][r] = 0;
      m[b] = kNegInf;
      lsum[b] = 0;
      mass[b] = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) wsum[b][u] = 0;
#pragma unroll
      for (int p = 0; p < KLQ; ++p) list[b][p] = Key<T>::sentinel();
    }
  }

  // ---------------------------------------------------------------- finalize
  const bool fin = a.n_split == 1;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int64_t i = qi[b];
    const int64_t prow = (int64_t)sp * a.N + i;
    if constexpr (CONS == C_LOGSUMEXP) {
      const T lt = F::gsum(lsum[b]);
      if (g == 0 && qv[b]) {
        const T mnat = m[b] * (T)kLn2 + ep[b];
        if (fin) {
          static_cast<T *>(bp.out)[i] = lt > (T)0 ? mnat + F::log(lt) : kNegInf;
        } else {
          T *pp = static_cast<T *>(bp.partial) + prow * 2;
          pp[0] = lt > (T)0 ? mnat : kNegInf;
          pp[1] = lt;
        }
      }
    } else if constexpr (CONS == C_SOFTMAX) {
      const T lt = F::gsum(lsum[b]);
      if (qv[b]) {
        const T inv = lt > (T)0 ? (T)1 / lt : (T)0;
        T *dst = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow * (a.C + 2) + 2;
        // A partial with no weight (l = 0) is skipped by the merge: its
        // values are not written.
        if (fin || lt > (T)0) {
#pragma unroll
          for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int r = 0; r < NREG; ++r) {
              const int ch = c * TM + F::key_of(r, g);
              if (ch < a.C) dst[ch] = fin ? o[b][c][r] * inv : o[b][c][r];
            }
        }
        // The row offset p_i drops out of the softmax but belongs to the
        // row's log-sum-exp: it rides on the partial maximum (the merge's
        // rescale is unchanged by a common shift).
        if (!fin && g == 0) {
          T *pp = static_cast<T *>(bp.partial) + prow * (a.C + 2);
          pp[0] = lt > (T)0 ? m[b] * (T)kLn2 + ep[b] : kNegInf;
          pp[1] = lt;
        }
        if (fin && g == 0 && bp.lse_out)
          static_cast<T *>(bp.lse_out)[i] = lt > (T)0 ? m[b] * (T)kLn2 + ep[b] + F::log(lt) : kNegInf;
      }
    } else if constexpr (NARROW) {
      T t = F::gsum((wsum[b][0] + wsum[b][1]) + (wsum[b][2] + wsum[b][3]));
      if (epi_post) t *= er[b];
      if (g == 0 && qv[b]) {
        T *dst = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow;
        dst[0] = t;
      }
    } else if constexpr (CONS == C_MATMUL) {
      if (qv[b]) {
        T *dst = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow * a.C;
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
          for (int r = 0; r < NREG; ++r) {
            const int ch = c * TM + F::key_of(r, g);
            if (ch < a.C) dst[ch] = o[b][c][r];
          }
      }
    } else if constexpr (CONS == C_DISPLACEMENT) {
      const T mt = F::gsum(mass[b]);
      if (qv[b]) {
        T *dst = fin ? static_cast<T *>(bp.out) + i * a.ldo : static_cast<T *>(bp.partial) + prow * a.D;
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
          for (int r = 0; r < NREG; ++r) {
            const int ch = c * TM + F::key_of(r, g);
            if (ch < a.D) dst[ch] = o[b][c][r] - Xp[i * a.ldx + ch] * mt;
          }
      }
    } else if constexpr (CONS == C_TOPK) {
      // Every lane group's list is its own partial (split sp, group g); the
      // merge kernel combines the n_split * G sorted lists of each row.
      if (qv[b]) {
        const int off = KLQ - a.k;
        const int64_t prow_g = ((int64_t)sp * G + g) * a.N + i;
#pragma unroll
        for (int p = 0; p < KLQ; ++p)
          if (p >= off) list[b][p].store(bp.partial, prow_g * a.k + (p - off));
      }
    }
  }
  }  // pass
}

// ------------------------------------------------------------------ dispatch

template <class T, int METRIC, int CONS, int DP, int CP, int KL>
hipError_t launch_mfma_kernel(const TileArgs &a, hipStream_t s) {
  const int slots = (a.mask.any && a.rb_pairs) ? a.rb_pairs : a.n_rb;
  dim3 grid((unsigned)(slots * a.n_split), 1, (unsigned)a.bat.n), block(MfmaShape<T, CONS, DP, CP, KL>::NT);
  if (a.mask.any) hipLaunchKernelGGL((mfma_tile<T, METRIC, CONS, DP, CP, KL, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((mfma_tile<T, METRIC, CONS, DP, CP, KL, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class T, int METRIC, int CONS, int DP>
hipError_t mfma_by_tile(const MfmaConfig &c, const TileArgs &a, hipStream_t s) {
  if constexpr (CONS == C_MATMUL || CONS == C_SOFTMAX) {
    if constexpr (CONS == C_MATMUL) {
      if (c.cp == 1) return launch_mfma_kernel<T, METRIC, CONS, DP, 1, 1>(a, s);
    }
    if constexpr (sizeof(T) == 8) {
      if (c.cp == 16) return launch_mfma_kernel<T, METRIC, CONS, DP, 16, 1>(a, s);
    }
    if (c.cp == 32) return launch_mfma_kernel<T, METRIC, CONS, DP, 32, 1>(a, s);
    if (c.cp == 64) return launch_mfma_kernel<T, METRIC, CONS, DP, 64, 1>(a, s);
  } else if constexpr (CONS == C_TOPK) {
    if (c.kl == 16) return launch_mfma_kernel<T, METRIC, CONS, DP, 1, 16>(a, s);
    if (c.kl == 64) return launch_mfma_kernel<T, METRIC, CONS, DP, 1, 64>(a, s);
  } else {
    return launch_mfma_kernel<T, METRIC, CONS, DP, 1, 1>(a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC, int DP>
hipError_t mfma_by_consumer(int consumer, const MfmaConfig &c, const TileArgs &a, hipStream_t s) {
  switch (consumer) {
    case C_MATMUL: return mfma_by_tile<T, METRIC, C_MATMUL, DP>(c, a, s);
    case C_DISPLACEMENT: return mfma_by_tile<T, METRIC, C_DISPLACEMENT, DP>(c, a, s);
    case C_LOGSUMEXP: return mfma_by_tile<T, METRIC, C_LOGSUMEXP, DP>(c, a, s);
    case C_SOFTMAX: return mfma_by_tile<T, METRIC, C_SOFTMAX, DP>(c, a, s);
    case C_TOPK: return mfma_by_tile<T, METRIC, C_TOPK, DP>(c, a, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int METRIC>
hipError_t mfma_launch_metric(int consumer, const MfmaConfig &c, const TileArgs &a, hipStream_t s) {
  switch (c.dp) {
    case 16: return mfma_by_consumer<T, METRIC, 16>(consumer, c, a, s);
    case 32: return mfma_by_consumer<T, METRIC, 32>(consumer, c, a, s);
    case 64: return mfma_by_consumer<T, METRIC, 64>(consumer, c, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pw
