// C ABI of the QSA sparse-prefill operator: host-side validation, then the
// gfx950 kernels. Every argument check happens before the first HIP call, so
// an invalid call enqueues nothing and writes nothing.

#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "qsa.h"
#include "qsa_internal.h"

namespace {

constexpr int64_t kMaxK = (int64_t)1 << 28; // idx rows are addressed with 32-bit byte offsets

bool aliases(const void *out, const void *lse, std::initializer_list<const void *> ins) {
    if (out == (const void *)lse) return true;
    for (const void *i : ins)
        if (i != nullptr && (i == out || i == (const void *)lse)) return true;
    return false;
}

// Checks shared by every entry point. `n_entries` is the index list length,
// `blk_shift` the log2 of the tokens one entry names.
qsa_status_t check_common(const void *q, const void *k, const void *v, const int32_t *idx, int64_t T,
                          int64_t n_kv_rows, int32_t Hq, int32_t Hkv, int32_t n_entries, int32_t blk_shift,
                          float scale, void *out, float *lse) {
    if (T < 0 || T > INT32_MAX || n_kv_rows < 0 || n_kv_rows > INT32_MAX) return QSA_ERR_INVALID_ARG;
    if (Hq < 1 || Hkv < 1 || n_entries < 0) return QSA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return QSA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return QSA_ERR_INVALID_ARG;
    if (T == 0) return QSA_OK;
    if (q == nullptr || out == nullptr || lse == nullptr) return QSA_ERR_INVALID_ARG;
    if (n_entries > 0 && idx == nullptr) return QSA_ERR_INVALID_ARG;
    // K/V rows are read only when there are some (a pool may be empty)
    if (n_entries > 0 && n_kv_rows > 0 && (k == nullptr || v == nullptr)) return QSA_ERR_INVALID_ARG;
    if (aliases(out, lse, {q, k, v, (const void *)idx})) return QSA_ERR_INVALID_ARG;
    if (n_kv_rows * (int64_t)Hkv > QSA_MAX_KV_ROWS) return QSA_ERR_UNSUPPORTED;
    if (((int64_t)n_entries << blk_shift) > kMaxK) return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

qsa_status_t run(const qsa::PrefillArgs &a, void *stream) {
    if (a.T == 0) return QSA_OK;
    return qsa::launch_prefill(a, (hipStream_t)stream);
}

qsa::PrefillArgs make_args(const void *q, const void *k, const void *v, const int32_t *idx, int64_t T,
                           int64_t n_kv_rows, int64_t q_pos0, int32_t Hq, int32_t Hkv, int32_t n_entries,
                           int32_t blk_shift, float scale, void *out, float *lse) {
    qsa::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.idx = idx;
    a.pool = false;
    a.q_pos = nullptr;
    a.slot_pos = nullptr;
    a.out = out;
    a.lse = lse;
    a.T = T;
    a.n_kv_rows = n_kv_rows;
    a.q_pos0 = q_pos0;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.K = n_entries;
    a.blk_shift = blk_shift;
    a.scale = scale;
    a.n_splits = 1;
    a.tiles_per_split = 0;
    a.workspace = nullptr;
    return a;
}

int log2_block(int32_t block_size) {
    for (int s = 0; s <= 4; ++s)
        if (block_size == (1 << s)) return s;
    return -1;
}

qsa_status_t sequence_call(const void *q, const void *k, const void *v, const int32_t *idx, int64_t T,
                           int64_t T_kv, int64_t q_pos0, int32_t Hq, int32_t Hkv, int32_t n_entries,
                           int32_t block_size, float scale, void *out, float *lse, void *stream) {
    const int shift = log2_block(block_size);
    if (shift < 0) return QSA_ERR_INVALID_ARG;
    // queries sit at q_pos0 .. q_pos0 + T - 1 and must lie inside the cache
    // (written without the sum, which could overflow)
    if (q_pos0 < 0 || T_kv < 0 || q_pos0 > T_kv || (T >= 0 && T > T_kv - q_pos0)) return QSA_ERR_INVALID_ARG;
    const qsa_status_t st = check_common(q, k, v, idx, T, T_kv, Hq, Hkv, n_entries, shift, scale, out, lse);
    if (st != QSA_OK || T == 0) return st;
    return run(make_args(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, n_entries, shift, scale, out, lse), stream);
}

// Checks of the decode entry points up to the workspace, and the call they
// make: `a` gets the arguments and split plan, `need` the workspace bytes the
// plan uses (0: no split). QSA_OK with n_req == 0 means nothing to do.
qsa_status_t decode_args(const void *q, const void *k_pool, const void *v_pool, const int32_t *slot_idx,
                         const int32_t *q_pos, const int32_t *slot_pos, int64_t n_req, int64_t n_slots, int32_t Hq,
                         int32_t Hkv, int32_t K, float scale, void *out, float *lse, qsa::PrefillArgs &a,
                         int64_t &need) {
    const qsa_status_t st =
        check_common(q, k_pool, v_pool, slot_idx, n_req, n_slots, Hq, Hkv, K, 0, scale, out, lse);
    if (st != QSA_OK || n_req == 0) return st;
    if (q_pos == nullptr || (slot_pos == nullptr && n_slots > 0)) return QSA_ERR_INVALID_ARG;
    if (aliases(out, lse, {(const void *)q_pos, (const void *)slot_pos})) return QSA_ERR_INVALID_ARG;
    const qsa::SplitPlan plan = qsa::plan_split(n_req, Hq, Hkv, K);
    need = qsa::split_workspace_bytes(n_req, Hq, plan);
    a = make_args(q, k_pool, v_pool, slot_idx, n_req, n_slots, 0, Hq, Hkv, K, 0, scale, out, lse);
    a.pool = true;
    a.q_pos = q_pos;
    a.slot_pos = slot_pos;
    a.n_splits = plan.n_splits;
    a.tiles_per_split = plan.tiles_per_split;
    a.workspace = nullptr;
    return QSA_OK;
}

} // namespace

namespace qsa {

SplitPlan plan_split(int64_t T, int32_t Hq, int32_t Hkv, int32_t K_slots) {
    // Aim for about 512 waves (two per CU). More ranges fill more of the GPU
    // but each range writes a 1 KB fp32 partial per head that the merge reads
    // back: measured on a 16-request (24, 2) K = 2,048 decode batch, 512
    // waves (16 ranges of 8 tiles) beat 256, 1,024, 2,048 and 4,096. Lists
    // are only cut when the unsplit launch has fewer than 256 waves.
    constexpr int64_t kTargetWaves = 512;
    const int64_t n_tiles = ((int64_t)K_slots + 15) / 16;
    const int64_t items = T * Hkv * (((int64_t)Hq / Hkv + 15) / 16);
    if (n_tiles <= 1 || items >= kTargetWaves / 2) return {1, (int32_t)n_tiles};
    int64_t tps = (n_tiles * items + kTargetWaves - 1) / kTargetWaves;
    if (tps < 1) tps = 1;
    return {(int32_t)((n_tiles + tps - 1) / tps), (int32_t)tps};
}

int64_t split_workspace_bytes(int64_t T, int32_t Hq, const SplitPlan &plan) {
    if (plan.n_splits <= 1) return 0;
    // per (row, head, range): a 16-byte (m, l, le) record and 256 fp32 of O.
    // Bounded for every size: a split happens only with items <= 255, each
    // item holds at most 16 heads, and n_splits <= 512 / items + 1, so there
    // are at most 16 * (512 + 255) partial rows (12.8 MB).
    return T * Hq * plan.n_splits * (16 + 256 * 4);
}

} // namespace qsa

extern "C" {

qsa_status_t qsa_sparse_prefill(const void *q, const void *k, const void *v, const int32_t *idx,
                                int64_t T, int32_t Hq, int32_t Hkv, int32_t K, float scale,
                                void *out, float *lse, void *stream) {
    return sequence_call(q, k, v, idx, T, T, 0, Hq, Hkv, K, 1, scale, out, lse, stream);
}

qsa_status_t qsa_sparse_prefill_extend(const void *q, const void *k, const void *v,
                                       const int32_t *idx, int64_t T, int64_t T_kv, int64_t q_pos0,
                                       int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out,
                                       float *lse, void *stream) {
    return sequence_call(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, K, 1, scale, out, lse, stream);
}

qsa_status_t qsa_sparse_prefill_blocks(const void *q, const void *k, const void *v,
                                       const int32_t *block_idx, int64_t T, int64_t T_kv,
                                       int64_t q_pos0, int32_t Hq, int32_t Hkv, int32_t n_blocks,
                                       int32_t block_size, float scale, void *out, float *lse,
                                       void *stream) {
    return sequence_call(q, k, v, block_idx, T, T_kv, q_pos0, Hq, Hkv, n_blocks, block_size, scale, out,
                         lse, stream);
}

qsa_status_t qsa_sparse_prefill_pool(const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *slot_idx, const int32_t *q_pos,
                                     const int32_t *slot_pos, int64_t total_q, int64_t n_slots,
                                     int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out,
                                     float *lse, void *stream) {
    const qsa_status_t st =
        check_common(q, k_pool, v_pool, slot_idx, total_q, n_slots, Hq, Hkv, K, 0, scale, out, lse);
    if (st != QSA_OK || total_q == 0) return st;
    if (q_pos == nullptr || (slot_pos == nullptr && n_slots > 0)) return QSA_ERR_INVALID_ARG;
    if (aliases(out, lse, {(const void *)q_pos, (const void *)slot_pos})) return QSA_ERR_INVALID_ARG;
    qsa::PrefillArgs a =
        make_args(q, k_pool, v_pool, slot_idx, total_q, n_slots, 0, Hq, Hkv, K, 0, scale, out, lse);
    a.pool = true;
    a.q_pos = q_pos;
    a.slot_pos = slot_pos;
    return run(a, stream);
}

int64_t qsa_sparse_decode_workspace_bytes(int64_t n_req, int32_t Hq, int32_t Hkv, int32_t K) {
    if (n_req < 0 || n_req > INT32_MAX || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || K < 0 || K > kMaxK) return -1;
    return qsa::split_workspace_bytes(n_req, Hq, qsa::plan_split(n_req, Hq, Hkv, K));
}

qsa_status_t qsa_sparse_decode(const void *q, const void *k_pool, const void *v_pool, const int32_t *slot_idx,
                               const int32_t *q_pos, const int32_t *slot_pos, int64_t n_req, int64_t n_slots,
                               int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out, float *lse,
                               void *workspace, int64_t workspace_bytes, void *stream) {
    qsa::PrefillArgs a;
    int64_t need = 0;
    qsa_status_t st = decode_args(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, n_req, n_slots, Hq, Hkv, K, scale,
                                  out, lse, a, need);
    if (st != QSA_OK || n_req == 0) return st;
    if (workspace_bytes < 0 || aliases(out, lse, {workspace})) return QSA_ERR_INVALID_ARG;
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0)
            return QSA_ERR_INVALID_ARG;
        for (const void *in : {q, k_pool, v_pool, (const void *)slot_idx, (const void *)q_pos,
                               (const void *)slot_pos})
            if (in == workspace) return QSA_ERR_INVALID_ARG;
        a.workspace = workspace;
    }
    return run(a, stream);
}

qsa_status_t qsa_sparse_decode_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                       const int32_t *slot_idx, const int32_t *q_pos, const int32_t *slot_pos,
                                       int64_t n_req, int64_t n_slots, int32_t Hq, int32_t Hkv, int32_t K,
                                       float scale, void *out, float *lse, void *stream) {
    qsa::PrefillArgs a;
    int64_t need = 0;
    qsa_status_t st = decode_args(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, n_req, n_slots, Hq, Hkv, K, scale,
                                  out, lse, a, need);
    if (st != QSA_OK || n_req == 0) return st;
    if (need > QSA_DECODE_SCRATCH_BYTES) return QSA_ERR_UNSUPPORTED;
    if (need > 0) {
        // the first HIP call of this entry point: every argument is checked
        st = qsa::device_scratch(&a.workspace);
        if (st != QSA_OK) return st;
    }
    return run(a, stream);
}

const char *qsa_status_string(qsa_status_t status) {
    switch (status) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported size";
    case QSA_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

} // extern "C"
