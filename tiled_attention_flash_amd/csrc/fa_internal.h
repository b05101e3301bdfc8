// fa_internal.h -- interface between the C-ABI front end (fa_host.cpp) and the
// kernel translation unit (fa_fwd_kernel.hip).  Not installed, not part of
// the ABI.
#pragma once

#include <stdint.h>

#include "fa.h"

namespace fa {

// Validated problem description handed to the launcher.  Sizes fit in int;
// every element offset derived from them fits in int64.
struct Problem {
    const void *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int B, L, H, Hkv, D;
    bool causal;
    float scale;
};

// Enqueues the forward kernels on `stream`.  Returns FA_OK or FA_ERR_LAUNCH.
int launch_forward(const Problem &p, hipStream_t stream);

}  // namespace fa
