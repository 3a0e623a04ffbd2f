// placeholder until the matrix-core MLP plan lands
#include "launch.h"
namespace ttt {
bool mlp_mfma_supported(int, int, int) { return false; }
hipError_t launch_mlp_mfma(const MlpArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace ttt
