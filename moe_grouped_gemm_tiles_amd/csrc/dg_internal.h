// dg_internal.h -- symbols libdg exports for its own tests, outside the C ABI
// of include/dg.h.
#pragma once

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

// Forces the width of the 256-row output tiles (256, 224 or 160 columns; 0 =
// chosen per call), so that tests can run every width on the same inputs.
// Process-wide; results agree with the automatic choice to the stated
// tolerance (the K order of every output is the same).  Other values ->
// DG_ERROR_INVALID_VALUE.
dg_status dg_internal_set_tile_n(int tile_n);

#ifdef __cplusplus
}
#endif
