// Backward tile kernels: double, rbf metric.
#include "grad_engine.h"

namespace pw {
hipError_t grad_launch_f64_rbf(int consumer, int side, int dt, int ct, const GradArgs &a, hipStream_t s) {
  return grad_launch_metric<double, M_RBF>(consumer, side, dt, ct, a, s);
}
hipError_t grad_topk_f64_rbf(int dt, const GradArgs &a, hipStream_t s) {
  return grad_topk_metric<double, M_RBF>(dt, a, s);
}
}  // namespace pw
