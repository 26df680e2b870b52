// Auxiliary kernels of libpw: the epilogue-vector pre-pass, row norms,
// output fills for empty reductions, and the merge of column-split partials.
#include "device_common.h"

namespace pw {

// ---------------------------------------------------------------------------
// Epilogue vectors: every program of the batch evaluated per element in
// double, rounded once to the dtype.
// ---------------------------------------------------------------------------
// Program blockIdx.y of the batch, for batch element blockIdx.z.
template <class T>
__global__ __launch_bounds__(256) void vec_prog_kernel(const VecProgBatch b) {
  const int pi = blockIdx.y;
  if (pi >= b.n_progs) return;
  const VecProg &p = b.p[pi];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= p.len) return;
  const int64_t z = blockIdx.z;
  double v = 0.0;
  for (int k = 0; k < p.n; ++k) {
    const VecInstr &in = p.ins[k];
    switch (in.op) {
      case VO_SET: v = in.c; break;
      case VO_MULC: v *= in.c; break;
      case VO_ADDC: v += in.c; break;
      case VO_MULV: v *= (double)ldg<T>(batch_ptr(in.v, in.bstride, z), e); break;
      case VO_ADDV: v += (double)ldg<T>(batch_ptr(in.v, in.bstride, z), e); break;
    }
  }
  static_cast<T *>(batch_ptr(p.out, p.out_bstride, z))[e] = (T)v;
}

hipError_t launch_vec_progs(int dtype, const VecProgBatch &b, int64_t n_batch, hipStream_t s) {
  int64_t len = 0;
  for (int i = 0; i < b.n_progs; ++i) len = b.p[i].len > len ? b.p[i].len : len;
  if (len == 0 || b.n_progs == 0) return hipSuccess;
  dim3 grid((unsigned)((len + 255) / 256), (unsigned)b.n_progs, (unsigned)n_batch), block(256);
  if (dtype == 0) hipLaunchKernelGGL(vec_prog_kernel<float>, grid, block, 0, s, b);
  else hipLaunchKernelGGL(vec_prog_kernel<double>, grid, block, 0, s, b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill a [rows, cols] block (leading dimension ld) with one value.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void fill_kernel(T *out, int64_t rows, int64_t cols, int64_t ld, T v) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * cols) return;
  out[(t / cols) * ld + t % cols] = v;
}

hipError_t launch_fill(int dtype, void *out, int64_t rows, int64_t cols, int64_t ld, double value, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0) hipLaunchKernelGGL(fill_kernel<float>, grid, block, 0, s, (float *)out, rows, cols, ld, (float)value);
  else hipLaunchKernelGGL(fill_kernel<double>, grid, block, 0, s, (double *)out, rows, cols, ld, value);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row means from row sums: out[b][i] = out[b][i] / c_i with c_i the kept
// count of row i (cnt[i], or M for every row when cnt is null); a row with
// c_i = 0 gets a quiet NaN. inv (optional) receives 1 / c_i, or 0 for an
// empty row, from batch element 0's threads. Device code is built without
// NaN semantics, so the NaN is chosen and stored as an integer bit pattern,
// out of the reach of float folding.
// ---------------------------------------------------------------------------
template <class T>
struct Bits;
template <>
struct Bits<float> {
  using U = uint32_t;
  static constexpr U kQuietNan = 0x7fc00000u;
};
template <>
struct Bits<double> {
  using U = uint64_t;
  static constexpr U kQuietNan = 0x7ff8000000000000ull;
};

template <class T>
__global__ __launch_bounds__(256) void mean_finish_kernel(T *out, int64_t N, int64_t total, const T *cnt, T M,
                                                          T *inv) {
  using U = typename Bits<T>::U;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t i = t % N;
  const T c = cnt ? cnt[i] : M;
  const bool kept = c > (T)0;
  const T q = out[t] / c;
  U b;
  __builtin_memcpy(&b, &q, sizeof b);
  reinterpret_cast<U *>(out)[t] = kept ? b : Bits<T>::kQuietNan;
  if (inv && t < N) inv[t] = kept ? (T)1 / c : (T)0;
}

hipError_t launch_mean_finish(int dtype, void *out, int64_t N, int64_t B, const void *cnt, int64_t M, void *inv,
                              hipStream_t s) {
  const int64_t n = N * B;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(mean_finish_kernel<float>, grid, block, 0, s, (float *)out, N, n, (const float *)cnt,
                       (float)M, (float *)inv);
  else
    hipLaunchKernelGGL(mean_finish_kernel<double>, grid, block, 0, s, (double *)out, N, n, (const double *)cnt,
                       (double)M, (double *)inv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Squared MMD from three row-sum vectors, one workgroup of 1024 threads per
// batch element: each thread keeps four independent double sums per vector
// (so four loads per vector are in flight, not one), the wave adds its lanes
// by butterfly, and the first wave adds the 16 waves' shares. The order is
// fixed for a given size, so the result is reproducible.
// ---------------------------------------------------------------------------
constexpr int kMmdFinishThreads = 1024;

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) v += __shfl_xor(v, sh, 64);
  return v;
}

template <class T>
__device__ inline double strided_sum(const T *p, int64_t n, int tid) {
  constexpr int S = kMmdFinishThreads;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int64_t i = tid;
  for (; i + 3 * S < n; i += 4 * S) {
    s0 += (double)p[i];
    s1 += (double)p[i + S];
    s2 += (double)p[i + 2 * S];
    s3 += (double)p[i + 3 * S];
  }
  for (; i < n; i += S) s0 += (double)p[i];
  return (s0 + s1) + (s2 + s3);
}

template <class T>
__global__ __launch_bounds__(kMmdFinishThreads) void mmd_finish_kernel(const T *rxx, const T *ryy, const T *rxy,
                                                                       int64_t n, int64_t m, double cx, double cy,
                                                                       double cxy, T *out) {
  constexpr int W = kMmdFinishThreads / 64;
  __shared__ double part[3][W];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double sx = wave_sum_f64(strided_sum(rxx + b * n, n, tid));
  double sxy = wave_sum_f64(strided_sum(rxy + b * n, n, tid));
  double sy = wave_sum_f64(strided_sum(ryy + b * m, m, tid));
  if (lane == 0) {
    part[0][wave] = sx;
    part[1][wave] = sy;
    part[2][wave] = sxy;
  }
  __syncthreads();
  if (wave == 0) {
    sx = lane < W ? part[0][lane] : 0.0;
    sy = lane < W ? part[1][lane] : 0.0;
    sxy = lane < W ? part[2][lane] : 0.0;
    sx = wave_sum_f64(sx);
    sy = wave_sum_f64(sy);
    sxy = wave_sum_f64(sxy);
    if (lane == 0) out[b] = (T)(cx * sx + cy * sy - cxy * sxy);
  }
}

hipError_t launch_mmd_finish(int dtype, const void *rxx, const void *ryy, const void *rxy, int64_t n, int64_t m,
                             int64_t B, double cx, double cy, double cxy, void *out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 grid((unsigned)B), block(kMmdFinishThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(mmd_finish_kernel<float>, grid, block, 0, s, (const float *)rxx, (const float *)ryy,
                       (const float *)rxy, n, m, cx, cy, cxy, (float *)out);
  else
    hipLaunchKernelGGL(mmd_finish_kernel<double>, grid, block, 0, s, (const double *)rxx, (const double *)ryy,
                       (const double *)rxy, n, m, cx, cy, cxy, (double *)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MMD gradient of one cloud for batch element b: the two sides of its
// within-cloud product (a, a2) and its side of the cross product (c),
// combined with the statistic's coefficients and scaled by G[b]; written,
// or added for a cloud shared by the batch.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void mmd_grad_combine_kernel(const T *a, const T *a2, const T *c, int64_t rows,
                                                               int64_t D, const T *G, int64_t b, double c1, double c2,
                                                               T *out, int64_t ldo, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * D) return;
  const int64_t i = t / D, d = t % D;
  const double v = (double)G[b] * (c1 * ((double)a[t] + (double)a2[t]) - c2 * (double)c[t]);
  T *o = out + i * ldo + d;
  *o = accumulate ? (T)((double)*o + v) : (T)v;
}

hipError_t launch_mmd_grad_combine(int dtype, const void *a, const void *a2, const void *c, int64_t rows, int64_t D,
                                   const void *G, int64_t b, double c1, double c2, void *out, int64_t ldo,
                                   bool accumulate, hipStream_t s) {
  const int64_t n = rows * D;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(mmd_grad_combine_kernel<float>, grid, block, 0, s, (const float *)a, (const float *)a2,
                       (const float *)c, rows, D, (const float *)G, b, c1, c2, (float *)out, ldo, (int)accumulate);
  else
    hipLaunchKernelGGL(mmd_grad_combine_kernel<double>, grid, block, 0, s, (const double *)a, (const double *)a2,
                       (const double *)c, rows, D, (const double *)G, b, c1, c2, (double *)out, ldo,
                       (int)accumulate);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Group ranges for the same_group mask: min and max id of each block of
// `block` consecutive entries (a row block, or a key tile), so the tile
// kernels can skip pairs of blocks whose ranges are disjoint. One wave per
// block: lanes read consecutive entries, then a butterfly reduction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_ranges_kernel(const int64_t *__restrict__ g, int64_t n, int block,
                                                           int64_t *__restrict__ out, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= nblocks) return;  // whole waves leave together
  const int64_t e0 = b * block, e1 = min(n, e0 + block);
  long long lo = g[e0], hi = g[e0];
  for (int64_t e = e0 + lane; e < e1; e += 64) {
    const long long v = g[e];
    lo = min(lo, v);
    hi = max(hi, v);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    lo = min(lo, (long long)__shfl_xor(lo, sh, 64));
    hi = max(hi, (long long)__shfl_xor(hi, sh, 64));
  }
  if (lane == 0) {
    out[2 * b] = lo;
    out[2 * b + 1] = hi;
  }
}

hipError_t launch_group_ranges(const int64_t *g, int64_t n, int block, int64_t *out, hipStream_t s) {
  const int64_t nb = (n + block - 1) / block;
  if (nb == 0) return hipSuccess;
  dim3 grid((unsigned)((nb + 3) / 4)), block_dim(256);
  hipLaunchKernelGGL(group_ranges_kernel, grid, block_dim, 0, s, g, n, block, out, nb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Spans of kept tiles: one workgroup per row block; its threads classify
// the key tiles with the tile kernels' own rule and reduce the first and the
// end column of the tiles not skipped. Runs after the group ranges it reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_spans_kernel(const MaskArgs m, int64_t N, int64_t M, int bm, int bn,
                                                         int64_t *__restrict__ out) {
  __shared__ unsigned long long s_first, s_end;
  const int rb = blockIdx.x;
  if (threadIdx.x == 0) {
    s_first = ~0ull;
    s_end = 0;
  }
  __syncthreads();
  const int64_t r0 = (int64_t)rb * bm, r1 = min(N, r0 + bm) - 1;
  const int64_t tiles = (M + bn - 1) / bn;
  unsigned long long first = ~0ull, end = 0;
  for (int64_t t = threadIdx.x; t < tiles; t += 256) {
    const int64_t j0 = t * bn, j1 = min(M, j0 + bn) - 1;
    if (tile_class(m, r0, r1, j0, j1, rb, t) == TILE_SKIP) continue;
    first = min(first, (unsigned long long)j0);
    end = max(end, (unsigned long long)(j1 + 1));
  }
  if (first != ~0ull) {
    atomicMin(&s_first, first);
    atomicMax(&s_end, end);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool none = s_first == ~0ull;
    out[2 * rb] = none ? 0 : (int64_t)s_first;
    out[2 * rb + 1] = none ? 0 : (int64_t)s_end;
  }
}

hipError_t launch_tile_spans(const MaskArgs &m, int64_t N, int64_t M, int bm, int bn, int n_rb, int64_t *out,
                             hipStream_t s) {
  if (n_rb == 0) return hipSuccess;
  dim3 grid((unsigned)n_rb), block(256);
  hipLaunchKernelGGL(tile_spans_kernel, grid, block, 0, s, m, N, M, bm, bn, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pair order of a masked launch: each row block's tile count as the paired
// launch deals it (band and span reach), sorted heaviest first with one
// workgroup's bitonic network in LDS (keys (~count, index), so ties keep
// index order and the order is deterministic). Pairing the i-th heaviest
// with the i-th lightest evens out pair totals that a sawtooth of packed
// sequences leaves uneven when blocks pair by index.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pair_order_kernel(const MaskArgs m, int64_t N, int64_t M, int bm, int bn,
                                                         int n_rb, int P, int *__restrict__ order) {
  __shared__ unsigned long long key[kMaxOrderedBlocks];
  for (int r = threadIdx.x; r < P; r += 256) {
    unsigned long long k = ~0ull;
    if (r < n_rb) {
      const int64_t r0 = (int64_t)r * bm, r1 = min(N, r0 + bm) - 1;
      int64_t f, l;
      band_range(m, r, r0, r1, 0, M, bn, &f, &l);
      const int64_t t = l > f ? (l - f + bn - 1) / bn : 0;
      k = ((unsigned long long)(0xffffffffu - (uint32_t)min(t, (int64_t)0xffffffff)) << 32) | (uint32_t)r;
    }
    key[r] = k;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const unsigned long long a = key[i], b = key[j];
          if (up ? (b < a) : (a < b)) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < n_rb; r += 256) order[r] = (int)(uint32_t)key[r];
}

hipError_t launch_pair_order(const MaskArgs &m, int64_t N, int64_t M, int bm, int bn, int n_rb, int *order,
                             hipStream_t s) {
  if (n_rb <= 0 || n_rb > kMaxOrderedBlocks) return hipErrorInvalidValue;
  int P = 1;
  while (P < n_rb) P <<= 1;
  hipLaunchKernelGGL(pair_order_kernel, dim3(1), dim3(256), 0, s, m, N, M, bm, bn, n_rb, P, order);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row norms |x_i|^2 for the kernels that evaluate distances through the
// expansion |x|^2 + |y|^2 - 2 x.y. L consecutive lanes share a row and read
// consecutive features, so a wave reads whole rows contiguously; the L
// partial sums are folded with lane exchanges inside the group.
// ---------------------------------------------------------------------------
template <class T, int L>
__global__ __launch_bounds__(256) void row_norms_kernel(const T *__restrict__ X_in, int64_t n, int64_t ld, int D,
                                                        T *__restrict__ out_in, bool inverse, int64_t x_bstride,
                                                        int64_t out_bstride) {
  const T *__restrict__ X = static_cast<const T *>(batch_ptr(X_in, x_bstride, blockIdx.y));
  T *__restrict__ out = static_cast<T *>(batch_ptr(out_in, out_bstride, blockIdx.y));
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / L;
  const int lane = (int)(t % L);
  T s = 0;
  if (row < n) {
    for (int d = lane; d < D; d += L) {
      const T v = X[row * ld + d];
      s = fma(v, v, s);
    }
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (row < n && lane == 0) out[row] = inverse ? (s > (T)0 ? (T)1 / sqrt(s) : (T)0) : s;
}

template <class T>
static hipError_t row_norms_t(const T *X, int64_t n, int64_t ld, int D, T *out, hipStream_t s, bool inv, int64_t nb,
                              int64_t xs, int64_t os) {
  dim3 block(256);
  auto grid = [&](int L) { return dim3((unsigned)((n * L + 255) / 256), (unsigned)nb); };
  if (D <= 4) hipLaunchKernelGGL((row_norms_kernel<T, 4>), grid(4), block, 0, s, X, n, ld, D, out, inv, xs, os);
  else if (D <= 8) hipLaunchKernelGGL((row_norms_kernel<T, 8>), grid(8), block, 0, s, X, n, ld, D, out, inv, xs, os);
  else hipLaunchKernelGGL((row_norms_kernel<T, 16>), grid(16), block, 0, s, X, n, ld, D, out, inv, xs, os);
  return hipGetLastError();
}

hipError_t launch_row_norms(int dtype, const void *X, int64_t n, int64_t ld, int D, void *out, hipStream_t s,
                            bool inverse, int64_t n_batch, int64_t x_bstride, int64_t out_bstride) {
  if (n == 0 || n_batch == 0) return hipSuccess;
  if (dtype == 0)
    return row_norms_t<float>((const float *)X, n, ld, D, (float *)out, s, inverse, n_batch, x_bstride, out_bstride);
  return row_norms_t<double>((const double *)X, n, ld, D, (double *)out, s, inverse, n_batch, x_bstride,
                             out_bstride);
}

// ---------------------------------------------------------------------------
// Merge of n_split column-split partials, always in split order 0..S-1 so
// results are deterministic for a fixed plan.
// ---------------------------------------------------------------------------
// The split merges read the partials kMergeBatch splits at a time, every
// load of a batch issued before any is used (a plain loop waits on each load
// in turn); the arithmetic and its order are a plain loop's: the maximum
// first, then the sums in split order.
constexpr int kMergeBatch = 8;

template <class T>
__global__ __launch_bounds__(256) void merge_sum_kernel(const TileArgs a, int W) {
  const BatchPtrs bp = batch_ptrs(a);
  // matmul (W = C) and displacement (W = D): plain sums of the partials.
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.N * W) return;
  const int64_t i = t / W;
  const int c = (int)(t % W);
  const T *part = static_cast<const T *>(bp.partial) + i * W + c;
  const int64_t stride = a.N * W;
  T s = 0;
  for (int s0 = 0; s0 < a.n_split; s0 += kMergeBatch) {
    T v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = s0 + u < a.n_split ? part[(s0 + u) * stride] : (T)0;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) s += v[u];
  }
  static_cast<T *>(bp.out)[i * a.ldo + c] = s;
}

template <class T>
__global__ __launch_bounds__(256) void merge_lse_kernel(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.N) return;
  const T *part = static_cast<const T *>(bp.partial) + i * 2;
  const int64_t stride = a.N * 2;
  const int n = a.n_split;
  T m = neg_inf<T>();
  for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
    T v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = s0 + u < n ? part[(s0 + u) * stride] : neg_inf<T>();
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) m = max(m, v[u]);
  }
  T l = 0;
  if (m != neg_inf<T>()) {
    for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
      T qm[kMergeBatch], ql[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        qm[u] = s0 + u < n ? part[(s0 + u) * stride] : (T)0;
        ql[u] = s0 + u < n ? part[(s0 + u) * stride + 1] : (T)0;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u)
        if (ql[u] > (T)0) l += ql[u] * dexp(qm[u] - m);
    }
  }
  static_cast<T *>(bp.out)[i] = (l > (T)0) ? m + dlog(l) : neg_inf<T>();
}

template <class T>
__global__ __launch_bounds__(256) void merge_softmax_kernel(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.N * a.C) return;
  const int64_t i = t / a.C;
  const int c = (int)(t % a.C);
  const int64_t W = a.C + 2;
  const T *part = static_cast<const T *>(bp.partial) + i * W;
  const int64_t stride = a.N * W;
  const int n = a.n_split;
  T m = neg_inf<T>();
  for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
    T v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) v[u] = s0 + u < n ? part[(s0 + u) * stride] : neg_inf<T>();
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) m = max(m, v[u]);
  }
  T l = 0, acc = 0;
  if (m != neg_inf<T>()) {
    for (int s0 = 0; s0 < n; s0 += kMergeBatch) {
      T qm[kMergeBatch], ql[kMergeBatch], qo[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const T *q = part + (s0 + u) * stride;
        qm[u] = s0 + u < n ? q[0] : (T)0;
        ql[u] = s0 + u < n ? q[1] : (T)0;
        qo[u] = s0 + u < n ? q[2 + c] : (T)0;
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (ql[u] > (T)0) {
          const T f = dexp(qm[u] - m);
          l += ql[u] * f;
          acc += qo[u] * f;
        }
      }
    }
  }
  static_cast<T *>(bp.out)[i * a.ldo + c] = (l > (T)0) ? acc / l : (T)0;
  // The split maxima carry the row offset, so m + log l is the row's lse.
  if (c == 0 && bp.lse_out) static_cast<T *>(bp.lse_out)[i] = (l > (T)0) ? m + dlog(l) : neg_inf<T>();
}

// Keep in `a` the KL smallest keys of two ascending lists a and b, ascending:
// min(a[p], b[KL-1-p]) is a bitonic sequence holding them, and log2(KL)
// half-cleaner stages sort it.
template <class T, int KL>
__device__ __forceinline__ void keep_smallest(Key<T> (&a)[KL], const Key<T> (&b)[KL]) {
#pragma unroll
  for (int p = 0; p < KL; ++p) a[p] = b[KL - 1 - p] < a[p] ? b[KL - 1 - p] : a[p];
#pragma unroll
  for (int j = KL / 2; j > 0; j >>= 1) {
#pragma unroll
    for (int p = 0; p < KL; ++p) {
      if ((p & j) == 0) {
        const bool sw = a[p + j] < a[p];
        const Key<T> lo = sw ? a[p + j] : a[p];
        const Key<T> hi = sw ? a[p] : a[p + j];
        a[p] = lo;
        a[p + j] = hi;
      }
    }
  }
}

// Each split left an ascending list of k keys per row. Lists of up to 16
// merge pairwise (keep_smallest), the next split's keys loaded before the
// current one is merged, so one row's loads are in flight together; longer
// lists take the keys one by one into a sorted list.
template <class T, int KL>
__global__ __launch_bounds__(256) void merge_topk_kernel(const TileArgs a) {
  const BatchPtrs bp = batch_ptrs(a);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.N) return;
  Key<T> list[KL];
#pragma unroll
  for (int p = 0; p < KL; ++p) list[p] = Key<T>::sentinel();
  if constexpr (KL <= 16) {
    Key<T> next[KL];
    auto load = [&](int sp) {
      const int64_t base = ((int64_t)sp * a.N + i) * a.k;
#pragma unroll
      for (int p = 0; p < KL; ++p) next[p] = p < a.k ? Key<T>::load(bp.partial, base + p) : Key<T>::sentinel();
    };
    load(0);
    for (int sp = 0; sp < a.n_split; ++sp) {
      Key<T> cur[KL];
#pragma unroll
      for (int p = 0; p < KL; ++p) cur[p] = next[p];
      if (sp + 1 < a.n_split) load(sp + 1);
      keep_smallest<T, KL>(list, cur);
    }
  } else {
    for (int sp = 0; sp < a.n_split; ++sp) {
      const int64_t base = ((int64_t)sp * a.N + i) * a.k;
      for (int p = 0; p < a.k; ++p) key_insert<T, KL>(list, Key<T>::load(bp.partial, base + p));
    }
  }
  T *v = static_cast<T *>(bp.out) + i * a.k;
  int64_t *ix = bp.idx + i * a.k;
#pragma unroll
  for (int p = 0; p < KL; ++p)
    if (p < a.k) {
      v[p] = list[p].value(a.largest);
      ix[p] = list[p].out_index();
    }
}

template <class T>
static hipError_t merge_t(int consumer, const TileArgs &a, hipStream_t s) {
  dim3 block(256);
  auto blocks = [&](int64_t n) { return dim3((unsigned)((n + 255) / 256), 1, (unsigned)a.bat.n); };
  if (a.N == 0) return hipSuccess;
  switch (consumer) {
    case C_MATMUL:
      hipLaunchKernelGGL(merge_sum_kernel<T>, blocks(a.N * a.C), block, 0, s, a, a.C);
      break;
    case C_DISPLACEMENT:
      hipLaunchKernelGGL(merge_sum_kernel<T>, blocks(a.N * a.D), block, 0, s, a, a.D);
      break;
    case C_LOGSUMEXP:
      hipLaunchKernelGGL(merge_lse_kernel<T>, blocks(a.N), block, 0, s, a);
      break;
    case C_SOFTMAX:
      hipLaunchKernelGGL(merge_softmax_kernel<T>, blocks(a.N * a.C), block, 0, s, a);
      break;
    case C_TOPK:
      if (a.k <= 8) hipLaunchKernelGGL((merge_topk_kernel<T, 8>), blocks(a.N), block, 0, s, a);
      else if (a.k <= 16) hipLaunchKernelGGL((merge_topk_kernel<T, 16>), blocks(a.N), block, 0, s, a);
      else hipLaunchKernelGGL((merge_topk_kernel<T, 64>), blocks(a.N), block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int consumer, const TileArgs &a, hipStream_t s) {
  return dtype == 0 ? merge_t<float>(consumer, a, s) : merge_t<double>(consumer, a, s);
}

}  // namespace pw
