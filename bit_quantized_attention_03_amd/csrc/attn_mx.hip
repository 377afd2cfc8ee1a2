// Microscaled FP4 / FP8 attention (placeholder until the kernel lands).
#include "device.hpp"
#include "kernels.hpp"

namespace sage {
hipError_t launch_attn_mx(const AttnArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sage
