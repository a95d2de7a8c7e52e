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
    if (n_entries > 0 && (k == nullptr || v == nullptr || idx == nullptr)) return QSA_ERR_INVALID_ARG;
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
    if (q_pos0 < 0 || T_kv < 0 || (T >= 0 && q_pos0 + T > T_kv)) return QSA_ERR_INVALID_ARG;
    const qsa_status_t st = check_common(q, k, v, idx, T, T_kv, Hq, Hkv, n_entries, shift, scale, out, lse);
    if (st != QSA_OK || T == 0) return st;
    return run(make_args(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, n_entries, shift, scale, out, lse), stream);
}

} // namespace

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
    if (q_pos == nullptr || slot_pos == nullptr) return QSA_ERR_INVALID_ARG;
    if (aliases(out, lse, {(const void *)q_pos, (const void *)slot_pos})) return QSA_ERR_INVALID_ARG;
    qsa::PrefillArgs a =
        make_args(q, k_pool, v_pool, slot_idx, total_q, n_slots, 0, Hq, Hkv, K, 0, scale, out, lse);
    a.q_pos = q_pos;
    a.slot_pos = slot_pos;
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
