// Matrix-core routing path (bf16, B*Tq >= 8): declarations shared with route.hip.
#pragma once

#include "launch.hpp"

namespace msa {

bool route_mfma_applicable(msa_dtype dt, int64_t B, int Tq, int Hkv, int D);
size_t route_mfma_workspace(msa_dtype dt, int64_t B, int Tq, int Hq, int Hkv, int D, int64_t N,
                            int num_cus);
hipError_t launch_route_mfma(const RouteArgs& a, const float* U, float* c, void* ws,
                             hipStream_t st);
// True when launch_route_mfma forms the unit-query sums itself (the
// route_mfma_kernel path with 16-byte aligned bf16 queries): the caller then
// need not run route_prep, and U is not read.
bool route_mfma_preps_itself(const RouteArgs& a);

}  // namespace msa
