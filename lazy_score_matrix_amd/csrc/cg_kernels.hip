// Vector steps of the conjugate-gradient solve of (S + shift I) A = B.
//
// Each CG iteration is one fused kernel product Q = S P (the tile engines)
// followed by these kernels over the [N, C] iterates (row-major, ld C):
//   pq         Q += shift P, and per-column partial sums of P.Q
//   scalars 1  alpha_c = rr_c / (p.q)_c             (one workgroup)
//   update     A += alpha P, R -= alpha Q, partial sums of R.R
//   scalars 2  beta_c = rr'_c / rr_c, convergence    (one workgroup)
//   direction  P = R + beta P
// Column sums are reduced in a fixed order (per block, then over blocks), so
// repeated solves are bitwise identical. Partials and scalars are double for
// both element types.
#include <algorithm>

#include "pw_internal.h"

namespace pw {
namespace {

constexpr int kCgThreads = 256;

__device__ __forceinline__ int cg_lanes_per_row(int C) {
  int ct = 1;
  while (ct < C && ct < 64) ct <<= 1;
  return ct;
}

// For every column c: the sum over this block's rows of f(i, c), reduced in
// a fixed tree over the row lanes and written to part[blockIdx.x * C + c].
// f may also update elements. Threads map to (row lane, column) so a wave
// reads consecutive columns of a row: coalesced for row-major [N, C].
template <class F>
__device__ void cg_block_sums(int64_t N, int C, double *part, F f) {
  __shared__ double sm[kCgThreads];
  const int t = threadIdx.x;
  const int ct = cg_lanes_per_row(C), rl = t / ct, ci = t % ct, nl = kCgThreads / ct;
  const int64_t r0 = (int64_t)blockIdx.x * kCgRows, r1 = min(N, r0 + kCgRows);
  for (int c0 = 0; c0 < C; c0 += ct) {
    const int c = c0 + ci;
    double acc = 0;
    if (c < C)
      for (int64_t i = r0 + rl; i < r1; i += nl) acc += f(i, c);
    sm[t] = acc;
    __syncthreads();
    for (int st = nl / 2; st >= 1; st >>= 1) {
      if (rl < st) sm[t] += sm[t + st * ct];
      __syncthreads();
    }
    if (rl == 0 && c < C) part[(int64_t)blockIdx.x * C + c] = sm[t];
    __syncthreads();
  }
}

template <class T>
__global__ __launch_bounds__(kCgThreads) void cg_init_kernel(const T *__restrict__ B, int64_t ldb, T *A, int64_t lda,
                                                             T *R, T *P, int64_t N, int C, double *part) {
  cg_block_sums(N, C, part, [&](int64_t i, int c) {
    const T b = B[i * ldb + c];
    A[i * lda + c] = 0;
    R[i * C + c] = b;
    P[i * C + c] = b;
    return (double)b * (double)b;
  });
}

template <class T>
__global__ __launch_bounds__(kCgThreads) void cg_pq_kernel(const T *__restrict__ P, T *Q, int64_t N, int C, T shift,
                                                           double *part) {
  cg_block_sums(N, C, part, [&](int64_t i, int c) {
    const T p = P[i * C + c];
    const T q = fma(shift, p, Q[i * C + c]);
    Q[i * C + c] = q;
    return (double)p * (double)q;
  });
}

template <class T>
__global__ __launch_bounds__(kCgThreads) void cg_update_kernel(const T *__restrict__ P, const T *__restrict__ Q, T *A,
                                                               int64_t lda, T *R, int64_t N, int C, CgState st,
                                                               double *part) {
  cg_block_sums(N, C, part, [&](int64_t i, int c) {
    const T al = (T)st.alpha[c];
    const T r = fma(-al, Q[i * C + c], R[i * C + c]);
    if (st.flag[c] == 1) {
      A[i * lda + c] = fma(al, P[i * C + c], A[i * lda + c]);
      R[i * C + c] = r;
    }
    return (double)r * (double)r;
  });
}

template <class T>
__global__ __launch_bounds__(kCgThreads) void cg_direction_kernel(const T *__restrict__ R, T *P, int64_t N, int C,
                                                                  CgState st) {
  const int64_t n = N * C;
  for (int64_t e = (int64_t)blockIdx.x * kCgThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kCgThreads) {
    const int c = (int)(e % C);
    if (st.flag[c] == 1) P[e] = fma((T)st.beta[c], P[e], R[e]);
  }
}

// One workgroup; each thread owns columns c = t, t + 256, ... and sums the
// block partials in block order.
__global__ __launch_bounds__(kCgThreads) void cg_scalars_kernel(int phase, const double *__restrict__ part, int nblk,
                                                                int C, CgState st, double tol2) {
  for (int c = threadIdx.x; c < C; c += kCgThreads) {
    double s = 0;
    for (int b = 0; b < nblk; ++b) s += part[(int64_t)b * C + c];
    if (phase == 0) {  // after init: s = |b_c|^2
      st.rr[c] = s;
      st.bb[c] = s;
      st.flag[c] = s > 0 ? 1 : 0;
    } else if (phase == 1) {  // s = p.(S + shift I)p
      if (st.flag[c] == 1 && !(s > 0)) st.flag[c] = 2;
      st.alpha[c] = st.flag[c] == 1 ? st.rr[c] / s : 0.0;
    } else if (st.flag[c] == 1) {  // s = |r'_c|^2
      st.beta[c] = s / st.rr[c];
      st.rr[c] = s;
      if (s <= tol2 * st.bb[c]) st.flag[c] = 0;
    }
  }
}

}  // namespace

int cg_blocks(int64_t N) { return (int)((N + kCgRows - 1) / kCgRows); }

hipError_t launch_cg_init(int dtype, const void *B, int64_t ldb, void *A, int64_t lda, void *R, void *P, int64_t N,
                          int C, double *part, hipStream_t s) {
  dim3 g(cg_blocks(N)), b(kCgThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(cg_init_kernel<float>, g, b, 0, s, (const float *)B, ldb, (float *)A, lda, (float *)R,
                       (float *)P, N, C, part);
  else
    hipLaunchKernelGGL(cg_init_kernel<double>, g, b, 0, s, (const double *)B, ldb, (double *)A, lda, (double *)R,
                       (double *)P, N, C, part);
  return hipGetLastError();
}

hipError_t launch_cg_pq(int dtype, const void *P, void *Q, int64_t N, int C, double shift, double *part,
                        hipStream_t s) {
  dim3 g(cg_blocks(N)), b(kCgThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(cg_pq_kernel<float>, g, b, 0, s, (const float *)P, (float *)Q, N, C, (float)shift, part);
  else
    hipLaunchKernelGGL(cg_pq_kernel<double>, g, b, 0, s, (const double *)P, (double *)Q, N, C, shift, part);
  return hipGetLastError();
}

hipError_t launch_cg_update(int dtype, const void *P, const void *Q, void *A, int64_t lda, void *R, int64_t N, int C,
                            CgState st, double *part, hipStream_t s) {
  dim3 g(cg_blocks(N)), b(kCgThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(cg_update_kernel<float>, g, b, 0, s, (const float *)P, (const float *)Q, (float *)A, lda,
                       (float *)R, N, C, st, part);
  else
    hipLaunchKernelGGL(cg_update_kernel<double>, g, b, 0, s, (const double *)P, (const double *)Q, (double *)A, lda,
                       (double *)R, N, C, st, part);
  return hipGetLastError();
}

hipError_t launch_cg_direction(int dtype, const void *R, void *P, int64_t N, int C, CgState st, hipStream_t s) {
  const int64_t n = N * C;
  dim3 g((unsigned)std::min<int64_t>((n + kCgThreads - 1) / kCgThreads, 4096)), b(kCgThreads);
  if (dtype == 0)
    hipLaunchKernelGGL(cg_direction_kernel<float>, g, b, 0, s, (const float *)R, (float *)P, N, C, st);
  else
    hipLaunchKernelGGL(cg_direction_kernel<double>, g, b, 0, s, (const double *)R, (double *)P, N, C, st);
  return hipGetLastError();
}

hipError_t launch_cg_scalars(int phase, const double *part, int nblk, int C, CgState st, double tol2,
                             hipStream_t s) {
  hipLaunchKernelGGL(cg_scalars_kernel, dim3(1), dim3(kCgThreads), 0, s, phase, part, nblk, C, st, tol2);
  return hipGetLastError();
}

}  // namespace pw
