// The library's switch for checking data-dependent preconditions before each launch.
#pragma once

#include <hip/hip_runtime_api.h>

namespace pkv {

// True when the environment variable PKV_DEBUG is set to a non-empty value other than "0"
// at the first call (read once per process).
bool debug_checks_enabled();

// True when the checks are enabled and `stream` is not recording a graph: a device call then
// runs its pkv_check_* on its device arrays before launching.
bool run_debug_checks(hipStream_t stream);

}  // namespace pkv
