// Backward tile kernels: float, linear metric.
#include "grad_engine.h"

namespace pw {
hipError_t grad_launch_f32_linear(int consumer, int side, int dt, int ct, const GradArgs &a, hipStream_t s) {
  return grad_launch_metric<float, M_LINEAR>(consumer, side, dt, ct, a, s);
}
hipError_t grad_topk_f32_linear(int dt, const GradArgs &a, hipStream_t s) {
  return grad_topk_metric<float, M_LINEAR>(dt, a, s);
}
}  // namespace pw
