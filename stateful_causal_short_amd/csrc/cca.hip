// CCA q/k conv (placeholder until the gfx950 kernel lands).
#include "common.hpp"
#include "kernels.hpp"
#include "cca.hpp"

namespace sc {
hipError_t launch_cca(const CcaArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sc
