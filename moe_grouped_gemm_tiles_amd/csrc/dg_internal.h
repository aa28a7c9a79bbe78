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

// The tile (bm x bn), K split (splits x slabs_per_split slabs of 128) and
// workspace bytes a dense call of this shape gets on a device with `cus` usable
// CUs.  Host arithmetic only.  Bad sizes or null outputs -> DG_ERROR_INVALID_VALUE.
dg_status dg_internal_dense_plan(int m, int n, int k, int cus, int* bm, int* bn, int* splits, int* slabs_per_split,
                                 size_t* ws_bytes);

#ifdef __cplusplus
}
#endif
