// Matrix-core routing path: not enabled yet; every shape takes the vector path.
#include "route_mfma.hpp"

namespace msa {

bool route_mfma_applicable(msa_dtype, int64_t, int, int, int) { return false; }
size_t route_mfma_workspace(msa_dtype, int64_t, int, int, int, int, int64_t, int) { return 0; }
hipError_t launch_route_mfma(const RouteArgs&, const float*, float*, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace msa
