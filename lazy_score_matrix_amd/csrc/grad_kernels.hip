// Backward support kernels: dispatch to the per-metric tile kernels, the
// fixed-order merge of the column-split partial gradients, and the softmax
// backward's per-row delta_i = G_i . O_i.
#include "pw_internal.h"

namespace pw {

#define PW_GRAD_DECL(dt, m)                                                                                  \
  hipError_t grad_launch_##dt##_##m(int consumer, int side, int dtile, int ct, const GradArgs &a,           \
                                    hipStream_t s);                                                          \
  hipError_t grad_topk_##dt##_##m(int dtile, const GradArgs &a, hipStream_t s);
PW_GRAD_DECL(f32, linear)
PW_GRAD_DECL(f32, sqeuclidean)
PW_GRAD_DECL(f32, rbf)
PW_GRAD_DECL(f32, cosine)
PW_GRAD_DECL(f64, linear)
PW_GRAD_DECL(f64, sqeuclidean)
PW_GRAD_DECL(f64, rbf)
PW_GRAD_DECL(f64, cosine)
#undef PW_GRAD_DECL

hipError_t grad_launch(int dtype, int metric, int consumer, int side, int dt, int ct, const GradArgs &a,
                       hipStream_t s) {
  if (dtype == 0) {
    switch (metric) {
      case M_LINEAR: return grad_launch_f32_linear(consumer, side, dt, ct, a, s);
      case M_SQEUCLIDEAN: return grad_launch_f32_sqeuclidean(consumer, side, dt, ct, a, s);
      case M_RBF: return grad_launch_f32_rbf(consumer, side, dt, ct, a, s);
      case M_COSINE: return grad_launch_f32_cosine(consumer, side, dt, ct, a, s);
    }
  } else {
    switch (metric) {
      case M_LINEAR: return grad_launch_f64_linear(consumer, side, dt, ct, a, s);
      case M_SQEUCLIDEAN: return grad_launch_f64_sqeuclidean(consumer, side, dt, ct, a, s);
      case M_RBF: return grad_launch_f64_rbf(consumer, side, dt, ct, a, s);
      case M_COSINE: return grad_launch_f64_cosine(consumer, side, dt, ct, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t grad_topk_launch(int dtype, int metric, int dt, const GradArgs &a, hipStream_t s) {
  if (dtype == 0) {
    switch (metric) {
      case M_LINEAR: return grad_topk_f32_linear(dt, a, s);
      case M_SQEUCLIDEAN: return grad_topk_f32_sqeuclidean(dt, a, s);
      case M_RBF: return grad_topk_f32_rbf(dt, a, s);
      case M_COSINE: return grad_topk_f32_cosine(dt, a, s);
    }
  } else {
    switch (metric) {
      case M_LINEAR: return grad_topk_f64_linear(dt, a, s);
      case M_SQEUCLIDEAN: return grad_topk_f64_sqeuclidean(dt, a, s);
      case M_RBF: return grad_topk_f64_rbf(dt, a, s);
      case M_COSINE: return grad_topk_f64_cosine(dt, a, s);
    }
  }
  return hipErrorInvalidValue;
}

namespace {

// One thread per (own row, slot): the sum over splits in split order, then
// the slot's destination: the own point's gradient, dV, or an op vector.
template <class T>
__global__ __launch_bounds__(256) void grad_merge_kernel(const T *__restrict__ part, int n_split, int64_t n_own,
                                                         int W, int D, int C1, GradOut o) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_own * W) return;
  const int64_t r = e / W;
  const int w = (int)(e % W);
  // Eight splits' partials at a time, every load of a batch issued before
  // any is used; the sum keeps split order.
  constexpr int NB = 8;
  const T *src = part + r * W + w;
  const int64_t stride = n_own * W;
  T acc = 0;
  for (int s0 = 0; s0 < n_split; s0 += NB) {
    T v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) v[u] = s0 + u < n_split ? src[(s0 + u) * stride] : (T)0;
#pragma unroll
    for (int u = 0; u < NB; ++u) acc += v[u];
  }
  if (w < D) {
    if (o.own) static_cast<T *>(o.own)[r * o.ld_own + w] = acc;
  } else if (w < D + C1) {
    if (o.dV) static_cast<T *>(o.dV)[r * o.lddv + (w - D)] = acc;
  } else {
    void *dst = o.dop[w - D - C1];
    if (dst) static_cast<T *>(dst)[r] = acc;
  }
}

template <class T>
__global__ __launch_bounds__(256) void grad_delta_kernel(const T *__restrict__ G, int64_t ldg, const T *__restrict__ O,
                                                         int64_t ldo, int64_t N, int C, T *delta) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  T acc = 0;
  for (int c = 0; c < C; ++c) acc = fma(G[i * ldg + c], O[i * ldo + c], acc);
  delta[i] = acc;
}

}  // namespace

hipError_t launch_grad_merge(int dtype, const GradArgs &a, int side, int64_t n_own, int C1, const GradOut &o,
                             hipStream_t s) {
  (void)side;
  const int64_t n = n_own * a.W;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(grad_merge_kernel<float>, grid, block, 0, s, (const float *)a.partial, a.n_split, n_own, a.W,
                       a.D, C1, o);
  else
    hipLaunchKernelGGL(grad_merge_kernel<double>, grid, block, 0, s, (const double *)a.partial, a.n_split, n_own,
                       a.W, a.D, C1, o);
  return hipGetLastError();
}

hipError_t launch_grad_delta(int dtype, const void *G, int64_t ldg, const void *O, int64_t ldo, int64_t N, int C,
                             void *delta, hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(grad_delta_kernel<float>, grid, block, 0, s, (const float *)G, ldg, (const float *)O, ldo, N,
                       C, (float *)delta);
  else
    hipLaunchKernelGGL(grad_delta_kernel<double>, grid, block, 0, s, (const double *)G, ldg, (const double *)O, ldo,
                       N, C, (double *)delta);
  return hipGetLastError();
}

}  // namespace pw
