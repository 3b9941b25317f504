// Backward kernels (placeholder until the MFMA backward lands).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace thd {

bool bwd_supported(int, int) { return false; }

int launch_bwd(const BwdParams&, int, int, void*) { return int(hipErrorNotSupported); }

}  // namespace thd
