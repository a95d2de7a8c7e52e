// Host-only check of the C ABI's argument validation, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer (any signed overflow,
// shift or out-of-bounds access in the validation aborts the program).
//
// The kernels are not linked: qsa::launch_prefill is replaced by a stub that
// receives every call the validation lets through and checks the invariants
// the kernels rely on (sizes in range, no 32-bit offset overflow, the pointers
// that will be read present, query positions inside the cache, split
// partials that fit the no-allocation decode's scratch), and
// qsa::device_scratch by one that returns a fake address. Pointers are
// never dereferenced, so fake non-null values are safe here. Every entry point
// is driven over the extremes of each argument and over a seeded random mix.
//
// Exit status 0 when every accepted call satisfies the invariants.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "qsa_internal.h"

namespace {

long g_launches = 0;
long g_scratch_lookups = 0;
long g_failures = 0;
bool g_sequence_call = false; // the current call is a sequence form (not pool)

void check(bool ok, const char *what) {
    if (!ok) {
        if (g_failures < 20) std::fprintf(stderr, "invariant violated: %s\n", what);
        ++g_failures;
    }
}

} // namespace

namespace qsa {

qsa_status_t launch_prefill(const PrefillArgs &a, hipStream_t) {
    ++g_launches;
    check(a.T >= 1 && a.T <= INT32_MAX, "1 <= T <= INT32_MAX");
    check(a.Hq >= 1 && a.Hkv >= 1 && a.Hq % a.Hkv == 0, "head counts");
    check(a.K >= 0, "K >= 0");
    check(a.blk_shift >= 0 && a.blk_shift <= 4, "block shift");
    check(((int64_t)a.K << a.blk_shift) <= ((int64_t)1 << 28), "slots per list <= 2^28");
    check(a.n_kv_rows >= 0 && a.n_kv_rows <= INT32_MAX, "K/V rows");
    check(a.n_kv_rows * (int64_t)a.Hkv <= QSA_MAX_KV_ROWS, "32-bit K/V byte offsets");
    check(std::isfinite(a.scale), "finite scale");
    check(a.q != nullptr && a.out != nullptr && a.lse != nullptr, "q, out, lse present");
    check(a.K == 0 || a.idx != nullptr, "indices present");
    check(a.K == 0 || a.n_kv_rows == 0 || (a.k != nullptr && a.v != nullptr), "k, v present");
    if (g_sequence_call) {
        check(!a.pool, "sequence call in sequence form");
        check(a.q_pos0 >= 0 && a.q_pos0 <= a.n_kv_rows - a.T, "queries inside the cache");
    } else {
        check(a.pool, "pool call in pool form");
        check(a.q_pos != nullptr, "q_pos present");
        check(a.n_kv_rows == 0 || a.slot_pos != nullptr, "slot_pos present");
    }
    if (a.n_splits > 1) {
        check(a.pool && a.workspace != nullptr && ((uintptr_t)a.workspace & 15u) == 0, "workspace");
        check(a.tiles_per_split >= 1, "tiles per range");
        check((int64_t)a.n_splits * a.tiles_per_split * 16 >= ((int64_t)a.K << a.blk_shift), "ranges cover the list");
        check(a.T * a.Hq * a.n_splits * 1040 <= QSA_DECODE_SCRATCH_BYTES, "split partials fit the static scratch");
    }
    return QSA_OK;
}

// the no-allocation decode's scratch: a fake, 256-byte aligned device address
qsa_status_t device_scratch(void **ptr) {
    ++g_scratch_lookups;
    *ptr = (void *)(uintptr_t)0x20000000u;
    return QSA_OK;
}

} // namespace qsa

namespace {

// distinct fake device addresses, 256-byte aligned, never dereferenced
void *P(int i) { return (void *)(uintptr_t)(0x10000000u + 0x1000u * (uintptr_t)i); }
const int32_t *PI(int i) { return (const int32_t *)P(i); }

const int64_t kI64[] = {INT64_MIN, -1, 0, 1, 3, 17, 256, 4096, 81920, 4194303, 4194304, (int64_t)INT32_MAX,
                        (int64_t)INT32_MAX + 1, INT64_MAX / 2, INT64_MAX};
const int32_t kI32[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 12, 16, 24, 255, 2048, 1 << 26, (1 << 28) + 1, INT32_MAX};
const float kScale[] = {0.0625f, 0.f, -1.f, std::numeric_limits<float>::quiet_NaN(),
                        std::numeric_limits<float>::infinity(), -std::numeric_limits<float>::infinity()};

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return g_rng;
}
template <typename T, size_t N> T pick(const T (&a)[N]) { return a[next() % N]; }

void *maybe_null(int i) { return next() % 8 == 0 ? nullptr : P(i); }

void call_all(int64_t T, int64_t T_kv, int64_t q_pos0, int32_t Hq, int32_t Hkv, int32_t K, int32_t bs,
              float scale, bool nulls) {
    void *q = nulls ? maybe_null(1) : P(1), *k = nulls ? maybe_null(2) : P(2), *v = nulls ? maybe_null(3) : P(3);
    const int32_t *idx = nulls && next() % 8 == 0 ? nullptr : PI(4);
    void *out = nulls ? maybe_null(5) : P(5);
    float *lse = (float *)(nulls ? maybe_null(6) : P(6));
    const int32_t *qp = nulls && next() % 8 == 0 ? nullptr : PI(7);
    const int32_t *sp = nulls && next() % 8 == 0 ? nullptr : PI(8);
    void *ws = nulls ? maybe_null(9) : P(9);
    g_sequence_call = true;
    (void)qsa_sparse_prefill(q, k, v, idx, T, Hq, Hkv, K, scale, out, lse, nullptr);
    (void)qsa_sparse_prefill_extend(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, K, scale, out, lse, nullptr);
    (void)qsa_sparse_prefill_blocks(q, k, v, idx, T, T_kv, q_pos0, Hq, Hkv, K, bs, scale, out, lse, nullptr);
    g_sequence_call = false;
    (void)qsa_sparse_prefill_pool(q, k, v, idx, qp, sp, T, T_kv, Hq, Hkv, K, scale, out, lse, nullptr);
    const int64_t need = qsa_sparse_decode_workspace_bytes(T, Hq, Hkv, K);
    const int64_t have = (int64_t)(next() % 3 == 0 ? 0 : (need > 0 ? need : 16));
    (void)qsa_sparse_decode(q, k, v, idx, qp, sp, T, T_kv, Hq, Hkv, K, scale, out, lse, ws, have, nullptr);
    (void)qsa_sparse_decode_noalloc(q, k, v, idx, qp, sp, T, T_kv, Hq, Hkv, K, scale, out, lse, nullptr);
}

} // namespace

int main() {
    // each argument over its extremes, the others at a valid default
    for (int64_t x : kI64) {
        call_all(x, 4096, 0, 12, 1, 64, 4, 0.0625f, false);
        call_all(64, x, 0, 12, 1, 64, 4, 0.0625f, false);
        call_all(64, 4096, x, 12, 1, 64, 4, 0.0625f, false);
    }
    for (int32_t x : kI32) {
        call_all(64, 4096, 0, x, 1, 64, 4, 0.0625f, false);
        call_all(64, 4096, 0, 24, x, 64, 4, 0.0625f, false);
        call_all(64, 4096, 0, 12, 1, x, 4, 0.0625f, false);
        call_all(64, 4096, 0, 12, 1, 64, x, 0.0625f, false);
    }
    for (float s : kScale) call_all(64, 4096, 0, 12, 1, 64, 4, s, false);
    // a seeded random mix of extremes, null pointers included
    for (int i = 0; i < 200000; ++i)
        call_all(pick(kI64), pick(kI64), pick(kI64), pick(kI32), pick(kI32), pick(kI32), pick(kI32), pick(kScale),
                 true);
    // a seeded mix of mostly valid sizes (one argument in ten an extreme), so
    // that many calls are accepted, including split decode plans
    const int32_t kBlock[] = {1, 2, 4, 8, 16};
    for (int i = 0; i < 200000; ++i) {
        const bool ext = next() % 10 == 0;
        // (the harness's own arithmetic saturates or wraps unsigned, so that
        // only the library's can trip the sanitizer)
        const int64_t T = ext && next() % 2 ? pick(kI64) : (int64_t)(1 + next() % 5000);
        const int64_t extra = (int64_t)(next() % 300000);
        const int64_t T_kv = ext && next() % 2 ? pick(kI64) : (T > INT64_MAX - extra ? T : T + extra);
        const uint64_t span = T_kv > T ? (uint64_t)T_kv - (uint64_t)T + 1u : 1u;
        const int64_t p0 = ext && next() % 2 ? pick(kI64) : (span ? (int64_t)(next() % span) : 0);
        const int32_t Hkv = ext && next() % 2 ? pick(kI32) : (int32_t)(1 + next() % 4);
        const int64_t hq = (int64_t)Hkv * (int64_t)(1 + next() % 40);
        const int32_t Hq = ext && next() % 2 ? pick(kI32)
                                              : (int32_t)(hq > INT32_MAX ? INT32_MAX : (hq < INT32_MIN ? INT32_MIN : hq));
        const int32_t K = ext && next() % 2 ? pick(kI32) : (int32_t)(next() % 5000);
        const int32_t bs = ext && next() % 2 ? pick(kI32) : pick(kBlock);
        call_all(T, T_kv, p0, Hq, Hkv, K, bs, ext && next() % 2 ? pick(kScale) : 0.0625f, next() % 4 == 0);
    }
    if (g_launches == 0) {
        std::fprintf(stderr, "no call was accepted: the harness exercised nothing\n");
        return 1;
    }
    if (g_scratch_lookups == 0) {
        std::fprintf(stderr, "no no-allocation decode call needed its scratch: the harness exercised nothing\n");
        return 1;
    }
    std::printf("%ld accepted calls checked (%ld scratch lookups), %ld invariant violations\n", g_launches,
                g_scratch_lookups, g_failures);
    return g_failures == 0 ? 0 : 1;
}
