// TTT-Linear prefill, MFMA path (bf16 storage, d = 64, mb = 16).
#include "common.hpp"
#include "launch.hpp"

namespace ttt {

bool linear_mfma_supported(const LinearArgs &) { return false; }
hipError_t launch_linear_mfma(const LinearArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace ttt
