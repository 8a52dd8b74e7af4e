// VALU chunk-score path: declarations shared with route.hip.
#pragma once

#include "launch.hpp"

namespace msa {

bool route_generic_supported(int Hkv);
// U[B*Tq][Hkv][D] (fp32) = per-group sums of the unit query heads.
hipError_t launch_route_prep(const RouteArgs& a, float* U, hipStream_t st);
// bf16, D = 128, B*Tq <= 4, Hkv in {4, 8, 16}: the coalesced streaming scan.
bool route_scan_fast_applicable(const RouteArgs& a);
hipError_t launch_route_scan_fast(const RouteArgs& a, const float* U, float* c, hipStream_t st);
// the streaming scan forms U from Qr itself (16-byte aligned Qr): no prep launch
bool route_scan_fast_preps_itself(const RouteArgs& a);
// any dtype and shape with Hkv <= 32: one thread per (query, chunk).
hipError_t launch_route_scan_generic(const RouteArgs& a, const float* U, float* c,
                                     hipStream_t st);

}  // namespace msa
