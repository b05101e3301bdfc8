// fa_internal.h -- interface between the C-ABI front end (fa_host.cpp) and the
// kernel translation units.  Not installed, not part of
// the ABI.
#pragma once

#include <stdint.h>

#include "fa.h"

namespace fa {

// Validated problem description handed to the launcher.  Sizes fit in int;
// every element offset derived from them fits in int64.
struct Problem {
    const void *q, *k, *v;  // k, v may be null when Lk == 0
    void *o;
    float *lse;  // may be null
    int B, Lq, Lk, H, Hkv, D;
    bool causal;
    int past_len;  // position of query row 0 among the keys (causal only); |past_len| <= 2^30
    float scale;
};

// Enqueues the forward kernels on `stream`.  Returns FA_OK or FA_ERR_LAUNCH.
int launch_forward(const Problem &p, hipStream_t stream);

// Forward on E4M3 inputs: q, k, v in p hold E4M3 codes, the value of a code
// is its descale factor times its E4M3 value.  Returns FA_OK, FA_ERR_SHAPE
// or FA_ERR_LAUNCH.
struct Fp8Descale {
    float q, k, v;
};
int launch_forward_fp8(const Problem &p, Fp8Descale ds, hipStream_t stream);

// Split-KV forward: bytes of fp32 workspace for rows_total = B*H*Lq output
// rows and n_splits key splits (-1 on overflow), and the launcher of the
// split kernel plus the merge kernel.  Returns FA_OK, FA_ERR_SHAPE or
// FA_ERR_LAUNCH.
int64_t splitkv_workspace_bytes(int64_t rows_total, int64_t n_splits, int D);
int launch_splitkv(const Problem &p, int n_splits, void *workspace, hipStream_t stream);

// The static scratch of the allocation-free split-KV entry point: its size,
// and its device address on the current device (looked up once per device).
// Returns FA_OK or FA_ERR_DEVICE.
constexpr int64_t kScratchBytes = FA_SPLITKV_SCRATCH_BYTES;
int splitkv_scratch(void **ptr);

// Validated backward problem.  Query row i sits at position i + past_len
// among the keys (causal only; 0 otherwise).
struct BwdProblem {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    float *delta;
    void *dq, *dk, *dv;
    int B, Lq, Lk, H, Hkv, D;
    bool causal;
    int past_len;
    float scale;
};

// Enqueues the backward kernels (Delta, dK/dV, dQ) on `stream`.  Returns
// FA_OK, FA_ERR_SHAPE or FA_ERR_LAUNCH.
int launch_backward(const BwdProblem &p, hipStream_t stream);

}  // namespace fa
