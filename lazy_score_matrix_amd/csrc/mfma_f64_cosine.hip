// Instantiates the MFMA tile engine for one dtype and metric.
#include "mfma_engine.h"

namespace pw {
template hipError_t mfma_launch_metric<double, M_COSINE>(int, const MfmaConfig &, const TileArgs &, hipStream_t);
}  // namespace pw
