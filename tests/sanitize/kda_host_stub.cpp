// Host-only stand-ins for the device side of libkda_mi355x.so, so that the
// C-ABI validation layer (kda_api.cpp) can be built with the host compiler's
// address and undefined-behaviour sanitizers and exercised on a machine
// without a GPU.  The *_plan entry points never reach these; the others
// report that no gfx950 device is present.
#include "../../gated_delta_rule_decode_amd/csrc/kda_internal.h"

namespace kda_detail {

int launch_recurrent(const RecParams &, const Launch &, void *) { return -9; }
int launch_fused(const FusedParams &, const Launch &, void *) { return -9; }
int launch_packed_fused(const PackedFusedParams &, const Launch &, void *) { return -9; }
int current_device_is_gfx950(int *device_out)
{
    if (device_out) *device_out = 0;
    return 0;
}
int device_is_gfx950(int) { return 0; }
int noalloc_scratch(void **) { return -9; }
const char *last_hip_error() { return "no device (host-only build)"; }

}  // namespace kda_detail
