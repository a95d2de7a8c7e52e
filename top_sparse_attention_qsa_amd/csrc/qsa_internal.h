// Internal interface between the C ABI shim (qsa_api.cpp) and the gfx950
// kernels (qsa_prefill.hip). Not installed; callers use include/qsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// One validated call of the sparse-prefill operator.
struct PrefillArgs {
    const void *q;           // bf16 [T, Hq, 256]
    const void *k;           // bf16 [n_kv_rows, Hkv, 256]
    const void *v;           // bf16 [n_kv_rows, Hkv, 256]
    const int32_t *idx;      // int32 [T, Hkv, K]
    bool pool;               // entries are pool slots (q_pos, slot_pos used)
    const int32_t *q_pos;    // pool form: int32 [T] query positions
    const int32_t *slot_pos; // pool form: int32 [n_kv_rows] slot positions (may be
                             // null when n_kv_rows == 0)
    void *out;               // bf16 [T, Hq, 256]
    float *lse;              // fp32 [T, Hq]
    int64_t T;               // query rows
    int64_t n_kv_rows;       // K/V rows: tokens of the sequence, or pool slots
    int64_t q_pos0;          // sequence modes: absolute position of query row 0
    int32_t Hq, Hkv;
    int32_t K;               // entries per index list
    int32_t blk_shift;       // an entry names 2^blk_shift tokens (0: token positions)
    float scale;
    int32_t n_splits;        // pool form: ranges each list is cut into (1: none)
    int32_t tiles_per_split; // 16-slot tiles per range
    void *workspace;         // n_splits > 1: split_workspace_bytes(...) bytes, 16-byte aligned
};

// How a list of K_slots slots is cut for T query rows so that the launch
// fills the GPU: every range holds tiles_per_split whole 16-slot tiles (the
// last may hold fewer), n_splits ranges in all.
struct SplitPlan {
    int32_t n_splits;
    int32_t tiles_per_split;
};
SplitPlan plan_split(int64_t T, int32_t Hq, int32_t Hkv, int32_t K_slots);

// Workspace bytes of a split launch (0 when n_splits == 1).
int64_t split_workspace_bytes(int64_t T, int32_t Hq, const SplitPlan &plan);

// Enqueue the operator on `stream`. Arguments are already validated and T > 0.
qsa_status_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// Device address of the current device's QSA_DECODE_SCRATCH_BYTES scratch
// array (looked up on the first call per device, then cached).
qsa_status_t device_scratch(void **ptr);

} // namespace qsa
