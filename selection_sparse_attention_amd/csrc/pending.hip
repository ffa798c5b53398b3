// Launchers of stages whose kernels live in their own files once written.
#include "args.hpp"

namespace sa {
hipError_t launch_pyramid(const PyramidArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_pyramid_select(const PyrSelectArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sa
