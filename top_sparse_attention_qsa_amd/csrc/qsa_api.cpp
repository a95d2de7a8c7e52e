// C ABI of the QSA sparse-prefill operator: host-side validation, then the
// gfx950 kernels. Every argument check happens before the first HIP call, so
// an invalid call enqueues nothing and writes nothing.

#include <math.h>
#include <stdint.h>

#include "qsa.h"
#include "qsa_internal.h"

namespace {

constexpr int64_t kMaxK = (int64_t)1 << 28; // idx rows are addressed with 32-bit byte offsets

qsa_status_t validate_and_launch(const void *q, const void *k, const void *v, const int32_t *idx,
                                 int64_t T, int64_t T_kv, int64_t q_pos0, int32_t Hq, int32_t Hkv,
                                 int32_t K, float scale, void *out, float *lse, void *stream) {
    if (T < 0 || T > INT32_MAX || T_kv < 0 || T_kv > INT32_MAX || q_pos0 < 0) return QSA_ERR_INVALID_ARG;
    if (Hq < 1 || Hkv < 1 || K < 0) return QSA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return QSA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return QSA_ERR_INVALID_ARG;
    if (q_pos0 + T > T_kv) return QSA_ERR_INVALID_ARG;
    if (T == 0) return QSA_OK;
    if (q == nullptr || out == nullptr || lse == nullptr) return QSA_ERR_INVALID_ARG;
    if (K > 0 && (k == nullptr || v == nullptr || idx == nullptr)) return QSA_ERR_INVALID_ARG;
    const void *outs[2] = {out, (const void *)lse};
    const void *ins[4] = {q, k, v, (const void *)idx};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o == i) return QSA_ERR_INVALID_ARG;
    if (out == (const void *)lse) return QSA_ERR_INVALID_ARG;
    if (T_kv * (int64_t)Hkv > QSA_MAX_KV_ROWS) return QSA_ERR_UNSUPPORTED;
    if ((int64_t)K > kMaxK) return QSA_ERR_UNSUPPORTED;

    qsa::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.idx = idx;
    a.out = out;
    a.lse = lse;
    a.T = T;
    a.T_kv = T_kv;
    a.q_pos0 = q_pos0;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.K = K;
    a.scale = scale;
    return qsa::launch_prefill(a, (hipStream_t)stream);
}

} // namespace

extern "C" {

qsa_status_t qsa_sparse_prefill(const void *q, const void *k, const void *v, const int32_t *idx,
                                int64_t T, int32_t Hq, int32_t Hkv, int32_t K, float scale,
                                void *out, float *lse, void *stream) {
    return validate_and_launch(q, k, v, idx, T, T, 0, Hq, Hkv, K, scale, out, lse, stream);
}

qsa_status_t qsa_sparse_prefill_extend(const void *q, const void *k, const void *v,
                                       const int32_t *idx, int64_t T, int64_t T_kv, int64_t q_pos0,
                                       int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out,
                                       float *lse, void *stream) {
    return validate_and_launch(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, K, scale, out, lse, stream);
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
