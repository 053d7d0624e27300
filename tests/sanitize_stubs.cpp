// Host-only stand-ins for the device launchers, for the sanitizer build of
// the planner and ABI layer (plan.cpp, api.cpp): every call that passes
// validation ends here and reports TRI_ERR_HIP, as a launch without a
// device would.
#include "tri_attn_internal.h"

namespace triattn {
int launch_attn_fwd(const AttnLaunch&, void*) { return fail(TRI_ERR_HIP, "host-only build: no device code"); }
int launch_split_merge(const AttnLaunch&, void*) { return fail(TRI_ERR_HIP, "host-only build: no device code"); }
int launch_dyn_plan(const DynLaunch&, void*) { return fail(TRI_ERR_HIP, "host-only build: no device code"); }
int launch_quantize_k(const QuantLaunch&, void*) { return fail(TRI_ERR_HIP, "host-only build: no device code"); }
int dyn_scratch(void**) { return fail(TRI_ERR_HIP, "host-only build: no device code"); }
}  // namespace triattn
