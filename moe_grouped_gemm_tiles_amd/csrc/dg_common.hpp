// dg_common.hpp -- host-side helpers shared by the translation units of libdg.
#pragma once

#include <hip/hip_runtime.h>

#include "dg.h"

namespace dg {

// Records the text of a failed HIP call for dg_last_hip_error() (per thread)
// and returns DG_ERROR_LAUNCH_FAILED.
dg_status record_hip_error(hipError_t e);

}  // namespace dg
