// Kernel-launcher stand-ins for host-only builds of the library's planner and
// C ABI (the sanitizer test links these instead of the HIP kernels): every
// launch reports an error, and no kernel shape is supported.
#include <hip/hip_runtime_api.h>

#include "internal.h"

namespace thd {
int launch_fwd(const FwdParams&, int, int, void*) { return int(hipErrorInvalidValue); }
int launch_fwd_pass(const FwdParams&, int, int, void*) { return int(hipErrorInvalidValue); }
int launch_bwd(const BwdParams&, int, int, void*) { return int(hipErrorInvalidValue); }
bool fwd_supported(int, int) { return false; }
bool bwd_supported(int, int) { return false; }
bool fwd_block_n_supported(int, int) { return false; }
int fwd_workgroups_per_cu(int) { return 1; }
int fwd_static_scratch(int, void**) { return int(hipErrorInvalidValue); }
}  // namespace thd
