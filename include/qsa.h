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
 * The device that holds the buffers must be the current HIP device, and
 * `stream` must belong to it; it is typed void * so that this header needs
 * no HIP include (pass a hipStream_t unchanged). Inputs are only read; out
 * and lse must not overlap any input or each other: the library rejects an
 * out or lse pointer equal to an input's (or to each other) but does not
 * detect partial overlaps, whose results are undefined. Calls on different
 * streams may run concurrently.
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
 * T * Hkv > QSA_MAX_KV_ROWS or K > 2^28.
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

/*
 * qsa_sparse_prefill_blocks -- the extend operation with indices that name
 * micro-blocks of block_size consecutive tokens instead of single tokens.
 * "Qwen4-Exp QSA llega al Ascend de Huawei", section "Por qué QSA es la parte
 * incómoda, en cifras", gives the model's indexer a compression ratio of 4 and
 * a budget of 2,048 selected micro-blocks per query; section "Nueve pruebas
 * que pasaron" tests the causal-tail remainders 0..3 at ratio 4. Entry b of a
 * list names tokens b*block_size .. b*block_size + block_size - 1, in that
 * order; each of those tokens s is used iff s <= q_pos0 + t (so a block that
 * straddles the query keeps only its past part). A negative entry masks its
 * whole block. The result equals qsa_sparse_prefill_extend on the expanded
 * token lists (n_blocks * block_size slots, blocks in list order).
 *
 *   block_idx   device pointer, int32 [T, Hkv, n_blocks]
 *   n_blocks    entries per list, >= 0
 *   block_size  1, 2, 4, 8 or 16 (1 is qsa_sparse_prefill_extend)
 *   others      as for qsa_sparse_prefill_extend
 *
 * Errors as for qsa_sparse_prefill_extend, plus QSA_ERR_INVALID_ARG for any
 * other block_size and QSA_ERR_UNSUPPORTED for n_blocks * block_size > 2^28.
 */
qsa_status_t qsa_sparse_prefill_blocks(const void *q, const void *k, const void *v,
                                       const int32_t *block_idx, int64_t T, int64_t T_kv,
                                       int64_t q_pos0, int32_t Hq, int32_t Hkv, int32_t n_blocks,
                                       int32_t block_size, float scale, void *out, float *lse,
                                       void *stream);

/*
 * qsa_sparse_prefill_pool -- a ragged batch of prefill requests over one
 * shared pool of K/V slots. "Qwen4-Exp QSA llega al Ascend de Huawei", section
 * "Nueve pruebas que pasaron": the indices are physical slots of the KV cache,
 * in no particular order, two requests may map a shared prefix to the same
 * slots, and cached content is reused. Query rows of all requests are
 * concatenated (total_q rows); each row carries its token position within its
 * own request, and each pool slot the position of the token it holds.
 *
 *   q, out       bf16 [total_q, Hq, 256];  lse fp32 [total_q, Hq]
 *   k_pool, v_pool  bf16 [n_slots, Hkv, 256]
 *   slot_idx     int32 [total_q, Hkv, K]: pool slots chosen for the row
 *   q_pos        int32 [total_q]: position of each query row in its request
 *   slot_pos     int32 [n_slots]: position of the token in each slot; a
 *                negative value marks a slot that holds no token
 *
 * Slot value s is used for query row r iff 0 <= s < n_slots and
 * 0 <= slot_pos[s] <= q_pos[r]; anything else is masked, never an error. The
 * slot lists are the indexer's and hold slots of the row's own request (the
 * pool itself does not record which request owns a slot). For one request
 * whose slots hold positions 0..n-1 this is qsa_sparse_prefill_extend with
 * the same lists after mapping slots to positions.
 *
 * Errors: QSA_ERR_INVALID_ARG for total_q < 0, n_slots < 0, either above
 * INT32_MAX, Hq < 1, Hkv < 1, K < 0, Hq % Hkv != 0, a non-finite scale, a
 * null pointer that would be used (q_pos is used whenever total_q > 0;
 * slot_pos, k_pool and v_pool may be NULL when n_slots == 0, every slot then
 * being masked) or out/lse equal to an input pointer;
 * QSA_ERR_UNSUPPORTED when n_slots * Hkv > QSA_MAX_KV_ROWS or K > 2^28.
 */
qsa_status_t qsa_sparse_prefill_pool(const void *q, const void *k_pool, const void *v_pool,
                                     const int32_t *slot_idx, const int32_t *q_pos,
                                     const int32_t *slot_pos, int64_t total_q, int64_t n_slots,
                                     int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out,
                                     float *lse, void *stream);

/*
 * qsa_sparse_decode -- one decode step of n_req requests over a K/V slot pool:
 * the pool form above with one query row per request (row r at position
 * q_pos[r] of request r). Decode is the serving phase the pages leave out of
 * their prefill path ("Qwen4-Exp QSA llega al Ascend de Huawei", section "Lo
 * que realmente añade la pull request"); the operation per row is exactly
 * qsa_sparse_prefill_pool's, and the results agree with it to rounding.
 *
 * With few requests there is too little work per list to fill the GPU, so
 * the library cuts each list into ranges of whole 16-slot tiles, computes the
 * ranges in parallel and merges them (a fixed order: results are
 * deterministic). The partials go to a caller-owned workspace of at least
 * qsa_sparse_decode_workspace_bytes(n_req, Hq, Hkv, K) bytes, 16-byte
 * aligned, device memory, overwritten by every call (calls sharing a
 * workspace must be ordered, e.g. on one stream). When that size is 0 the
 * workspace is not used and may be NULL.
 *
 *   arguments as for qsa_sparse_prefill_pool with total_q = n_req, plus
 *   workspace, workspace_bytes
 *
 * Errors as for qsa_sparse_prefill_pool, plus QSA_ERR_INVALID_ARG for a
 * workspace that is needed but NULL, smaller than required, not 16-byte
 * aligned, or equal to another argument's pointer.
 *
 * qsa_sparse_decode_workspace_bytes returns -1 for sizes qsa_sparse_decode
 * would refuse: n_req < 0 or above INT32_MAX, Hq < 1, Hkv < 1,
 * Hq % Hkv != 0, K < 0 or K > 2^28.
 */
int64_t qsa_sparse_decode_workspace_bytes(int64_t n_req, int32_t Hq, int32_t Hkv, int32_t K);
qsa_status_t qsa_sparse_decode(const void *q, const void *k_pool, const void *v_pool, const int32_t *slot_idx,
                               const int32_t *q_pos, const int32_t *slot_pos, int64_t n_req, int64_t n_slots,
                               int32_t Hq, int32_t Hkv, int32_t K, float scale, void *out, float *lse,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * qsa_sparse_decode_noalloc -- qsa_sparse_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same operation, kernels and results,
 * bit for bit, with the split partials in a scratch array that the library
 * holds in device memory instead of a caller's workspace. The call allocates
 * nothing.
 *
 * The scratch is QSA_DECODE_SCRATCH_BYTES (16 MiB) per GPU, held from the
 * library's load until the process ends; the first call on a device looks up
 * that device's copy (a runtime query that may load the library's code on that
 * device), so make one call on each device before capturing calls in a HIP
 * graph. Every valid size fits it: the split plan never needs
 * more than about 12.8 MB (at most 16 * 767 partial rows of 1,040 bytes).
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (e.g. on two streams at once) race and give undefined results;
 * calls ordered on one stream are safe. Nothing in the scratch needs to
 * start at zero: each call writes every partial it reads.
 *
 *   arguments as for qsa_sparse_decode, without workspace / workspace_bytes
 *
 * Errors as for qsa_sparse_decode (minus the workspace checks), plus
 * QSA_ERR_UNSUPPORTED if a split plan ever needed more than
 * QSA_DECODE_SCRATCH_BYTES (no valid size does) or the current device
 * number is 64 or higher, and QSA_ERR_LAUNCH if the HIP runtime cannot give
 * the scratch's device address.
 */
#define QSA_DECODE_SCRATCH_BYTES (16LL << 20)
qsa_status_t qsa_sparse_decode_noalloc(const void *q, const void *k_pool, const void *v_pool,
                                       const int32_t *slot_idx, const int32_t *q_pos, const int32_t *slot_pos,
                                       int64_t n_req, int64_t n_slots, int32_t Hq, int32_t Hkv, int32_t K,
                                       float scale, void *out, float *lse, void *stream);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char *qsa_status_string(qsa_status_t status);

/* ABI revision of this header; bumped on any incompatible change. */
#define QSA_ABI_VERSION 3
int32_t qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
