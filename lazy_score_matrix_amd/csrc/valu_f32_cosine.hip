// Instantiates the generic VALU tile engine for one dtype and metric.
#include "valu_engine.h"

namespace pw {
template hipError_t valu_launch_metric<float, M_COSINE>(int, const ValuConfig &, const TileArgs &, hipStream_t);
}  // namespace pw
