// Internal interface between the C ABI shim (qsa_api.cpp) and the gfx950
// kernels (qsa_prefill.hip). Not installed; callers use include/qsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// One validated call of the sparse-prefill operator.
struct PrefillArgs {
    const void *q;      // bf16 [T, Hq, 256]
    const void *k;      // bf16 [T_kv, Hkv, 256]
    const void *v;      // bf16 [T_kv, Hkv, 256]
    const int32_t *idx; // int32 [T, Hkv, K]
    void *out;          // bf16 [T, Hq, 256]
    float *lse;         // fp32 [T, Hq]
    int64_t T;          // query rows
    int64_t T_kv;       // K/V rows
    int64_t q_pos0;     // absolute position of query row 0
    int32_t Hq, Hkv, K;
    float scale;
};

// Enqueue the operator on `stream`. Arguments are already validated and T > 0.
qsa_status_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

} // namespace qsa
