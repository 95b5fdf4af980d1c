// Declarations shared between the library's own source files (not part of
// the C ABI).
#ifndef SATTN_INTERNAL_H
#define SATTN_INTERNAL_H

#include <hip/hip_runtime.h>

// The split-key forward for problems too small to fill the chip: arguments
// as sattn_fwd (already validated), enqueued on `stream`; with `vrows` the
// third array is V as rows [Hkv][T][64] (as sattn_fwd_vrows) instead of V^T.
void sattn_fwd_split_launch(const void* Q, const void* K, const void* V, void* O, float* L,
                            float c, int T, int Hq, int Hkv, bool vrows, hipStream_t stream);

#include "sattn_check.h"

#endif  // SATTN_INTERNAL_H
