/*
 * qsa.h -- C ABI of the QSA sparse-attention prefill operator for MI355X (gfx950).
 *
 * The operation is the one described in "Qwen4-Exp QSA llega al Ascend de
 * Huawei: dentro del PR de prefill CANN opcional de SGLang" (orcarouter.ai,
 * Spanish page), section "Lo que realmente añade la pull request": for each
 * query token t and query head h, attention over only the token positions an
 * upstream indexer selected for (t, KV head of h),
 *
 *     out[t,h,:] = sum_j softmax_j(scale * q[t,h,:] . k[s_j,g,:]) * v[s_j,g,:]
 *     lse[t,h]   = ln sum_j exp(scale * q[t,h,:] . k[s_j,g,:])
 *
 * with g = h / (Hq / Hkv) (contiguous groups of query heads share a KV head),
 * the head-dim-256 scale 1/sqrt(256) kept by default, -1 slots masked and a
 * fully masked row producing a zero output. The same page's section "Nueve
 * pruebas que pasaron" lists the cases this ABI covers: unordered physical
 * slots, selection widths 1/63/64/65/2051, default and explicit scales, fully
 * masked rows, zero selection width, non-contiguous inputs (made contiguous by
 * the caller), causal tails.
 *
 * Causality: a slot value s is used iff 0 <= s <= t, where t is the query's
 * absolute position. Every other value (-1, any negative, a future position)
 * is masked; index values are never an error. A position listed twice counts
 * as two softmax terms.
 *
 * Layouts: every tensor is device memory, contiguous, row-major:
 *     q    bf16  [T, Hq, 256]
 *     k, v bf16  [T_kv, Hkv, 256]
 *     idx  int32 [T, Hkv, K]
 *     out  bf16  [T, Hq, 256]        (written)
 *     lse  fp32  [T, Hq]             (written; -inf for an empty row)
 * bf16 is passed as raw 16-bit storage (const void *). Results: out is the
 * fp32-accumulated value rounded to nearest even; an empty row gets +0.0 and
 * lse = -inf.
 *
 * Ownership and execution: the caller owns every buffer. The library keeps no
 * allocation and no per-call state; it enqueues its kernels on `stream` (a
 * hipStream_t, NULL for the null stream) and returns without synchronising.
 * Inputs are only read; out and lse must not overlap any input or each other.
 * Calls on different streams may run concurrently.
 *
 * Errors: arguments are validated on the host before any HIP call; on error
 * nothing is enqueued and nothing is written. A failed kernel launch returns
 * QSA_ERR_LAUNCH. Faults inside a kernel surface asynchronously through the
 * HIP runtime, as for any kernel.
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, non-finite scale */
    QSA_ERR_UNSUPPORTED = 2, /* valid but outside the kernel's limits (see each entry point) */
    QSA_ERR_LAUNCH = 3       /* the HIP runtime refused the kernel launch */
} qsa_status_t;

/* Head dimension fixed by the operator (bf16, 256). */
#define QSA_HEAD_DIM 256

/* Largest T_kv * Hkv accepted: K and V rows are addressed with 32-bit byte
 * offsets, T_kv * Hkv * 512 must stay below 2^31. */
#define QSA_MAX_KV_ROWS 4194303LL

/*
 * qsa_sparse_prefill -- one prefill sequence of T tokens, query row t at
 * position t, K/V of the same T tokens.
 *
 *   q, k, v   device pointers, layouts above (T_kv = T)
 *   idx       device pointer, int32 [T, Hkv, K]; may be NULL when K == 0
 *   T         tokens, 0 <= T <= INT32_MAX; T == 0 is a no-op returning QSA_OK
 *   Hq, Hkv   query and KV heads, both >= 1, Hq % Hkv == 0 (any group size)
 *   K         selection width (slots per (t, KV head)), K >= 0; K == 0 makes
 *             every row empty
 *   scale     logit scale, finite (1/16 = 1/sqrt(256) is the model's)
 *   out, lse  device pointers, written
 *   stream    hipStream_t
 *
 * Returns QSA_ERR_INVALID_ARG for a null pointer that would be used, T < 0,
 * T > INT32_MAX, Hq < 1, Hkv < 1, K < 0, Hq % Hkv != 0, a non-finite scale or
 * out/lse equal to an input pointer; QSA_ERR_UNSUPPORTED when
 * T * Hkv > QSA_MAX_KV_ROWS.
 */
qsa_status_t qsa_sparse_prefill(const void *q, const void *k, const void *v, const int32_t *idx,
                                int64_t T, int32_t Hq, int32_t Hkv, int32_t K, float scale,
                                void *out, float *lse, void *stream);

/*
 * qsa_sparse_prefill_extend -- the same operation for T query tokens that
 * extend a sequence whose first q_pos0 tokens are already cached: query row t
 * sits at absolute position q_pos0 + t and K/V hold T_kv >= q_pos0 + T rows.
 * This is the long-prefill case of "Qwen4-Exp QSA llega al Ascend de Huawei",
 * section "Nueve pruebas que pasaron" (queries against a longer KV cache).
 * A slot value s is used iff 0 <= s <= q_pos0 + t.
 *
 *   q, idx, out, lse have T rows; k and v have T_kv rows.
 *   q_pos0 >= 0, T_kv >= q_pos0 + T, T_kv * Hkv <= QSA_MAX_KV_ROWS.
 *
 * qsa_sparse_prefill(...) equals qsa_sparse_prefill_extend(..., T_kv = T,
 * q_pos0 = 0, ...). Errors as for qsa_sparse_prefill, plus
 * QSA_ERR_INVALID_ARG for q_pos0 < 0 or T_kv < q_pos0 + T.
 */
qsa_status_t qsa_sparse_prefill_extend(const void *q, const void *k, const void *v,
                                       const int32_t *idx, int64_t T, int64_t T_kv, int64_t q_pos0,
                                       int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out,
                                       float *lse, void *stream);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char *qsa_status_string(qsa_status_t status);

/* ABI revision of this header; bumped on any incompatible change. */
#define QSA_ABI_VERSION 1
int32_t qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
