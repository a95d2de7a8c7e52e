// Measured ceiling of a random-row gather on this GPU, with the operator's
// load shape: every 16-byte-per-lane buffer load covers two whole 512-byte
// rows (lane l reads chunk l & 31 of row 2i + (l >> 5)), the rows are chosen
// at random (one pair per instruction, the same in every lane of the wave),
// and each wave keeps `loads` such loads in flight continuously: it folds the
// oldest one's data into a register and issues the next in its place, as the
// operator's kernel does. Nothing else runs: no LDS, no MFMA. The buffer size decides
// where the rows come from (a few MB: the L2s; tens to hundreds of MB: the
// Infinity Cache; GBs: HBM), and dynamic LDS fixes the waves per CU.
//
// It is a measuring tool beside the benchmark, not part of the operator. Every
// access stays inside the buffer (row < rows, chunk offset <= 496), which the
// buffer descriptor's range check enforces as well.
//
//   qsa_gather_probe <rows> <waves_per_cu: 4|8|12|16> <iterations> <loads: 8|16|24|32> [repeats] [far_permille]
// prints one line: the median over `repeats` timed launches of the bytes the
// waves received per second. With far_permille < 1000, each row pair comes
// from the whole buffer with that probability and otherwise from its first
// 8,192 rows (4 MB, which the L2s hold): a given mix of L2 hits and misses.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int NL>
__global__ __launch_bounds__(256) void gather_probe(const uint8_t *buf, uint32_t rows, uint32_t hot_rows,
                                                    uint32_t far_permille, uint32_t iters, uint32_t *out) {
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)buf, 0, (int)(rows * 512u), 0x00020000);
    uint32_t s = wave * 2654435761u + 12345u; // wave-uniform LCG state
    const uint32_t chunk = (uint32_t)(lane & 31) * 16u;
    const bool upper = (lane >> 5) != 0;
    auto next = [&]() -> u32x4_t {
        // a pair of rows from the whole buffer with probability far_permille /
        // 1000, otherwise from its first hot_rows rows
        // (a row index is the high half of state x span: no division)
        s = s * 1664525u + 1013904223u;
        const uint32_t span = __umulhi(s, 1000u) < far_permille ? rows : hot_rows;
        s = s * 1664525u + 1013904223u;
        const uint32_t r0 = __umulhi(s, span);
        s = s * 1664525u + 1013904223u;
        const uint32_t r1 = __umulhi(s, span);
        return __builtin_amdgcn_raw_buffer_load_b128(r, (upper ? r1 : r0) * 512u + chunk, 0, 0);
    };
    // a rolling window of NL loads: each step folds the oldest load's data
    // into the accumulator and issues a new load in its place, so NL - 1 to NL
    // loads stay in flight all the time (loads return in order)
    u32x4_t v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = next();
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            acc ^= v[i];
            v[i] = next();
            // keep each step's load where it is (not gathered into a burst)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) acc ^= v[i];
    out[(size_t)wave * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

static int fail(const char *what, hipError_t e) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
}

int main(int argc, char **argv) {
    if (argc < 5) {
        fprintf(stderr, "usage: %s rows waves_per_cu iterations loads [repeats]\n", argv[0]);
        return 2;
    }
    const long rows_l = atol(argv[1]);
    const int wpc = atoi(argv[2]);
    const long iters_l = atol(argv[3]);
    const int nl = atoi(argv[4]);
    const int repeats = argc > 5 ? atoi(argv[5]) : 5;
    const long far_l = argc > 6 ? atol(argv[6]) : 1000;
    if (rows_l < 2 || rows_l * 512L >= (1L << 31) || iters_l < 1 || iters_l > 100000 || repeats < 1 ||
        repeats > 50 || (wpc != 4 && wpc != 8 && wpc != 12 && wpc != 16) ||
        (nl != 8 && nl != 16 && nl != 24 && nl != 32) || far_l < 0 || far_l > 1000) {
        fprintf(stderr, "argument out of range\n");
        return 2;
    }
    const uint32_t rows = (uint32_t)rows_l, iters = (uint32_t)iters_l, far = (uint32_t)far_l;
    const uint32_t hot = rows < 8192u ? rows : 8192u;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, 0);
    if (e != hipSuccess) return fail("hipGetDeviceProperties", e);
    // four rounds of the resident waves, in 4-wave blocks
    const uint32_t blocks = (uint32_t)prop.multiProcessorCount * (uint32_t)wpc;
    // dynamic LDS caps the 4-wave blocks per CU (160 KB of LDS per CU)
    const size_t lds = wpc == 4 ? 81 * 1024 : wpc == 8 ? 60 * 1024 : wpc == 12 ? 50 * 1024 : 36 * 1024;
    auto kern = nl == 8 ? gather_probe<8> : nl == 16 ? gather_probe<16> : nl == 24 ? gather_probe<24> : gather_probe<32>;
    uint8_t *buf = nullptr;
    uint32_t *out = nullptr;
    if ((e = hipMalloc(&buf, (size_t)rows * 512)) != hipSuccess) return fail("hipMalloc", e);
    if ((e = hipMalloc(&out, (size_t)blocks * 4 * 64 * sizeof(uint32_t))) != hipSuccess) return fail("hipMalloc", e);
    if ((e = hipMemset(buf, 1, (size_t)rows * 512)) != hipSuccess) return fail("hipMemset", e);
    hipEvent_t e0, e1;
    if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess)
        return fail("hipEventCreate", e);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, 0, (const uint8_t *)buf, rows, hot, far, 2u, out);
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail("warm-up", e);
    std::vector<float> ms(repeats);
    for (int rep = 0; rep < repeats; ++rep) {
        (void)hipEventRecord(e0, 0);
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, 0, (const uint8_t *)buf, rows, hot, far, iters, out);
        (void)hipEventRecord(e1, 0);
        if ((e = hipEventSynchronize(e1)) != hipSuccess) return fail("launch", e);
        (void)hipEventElapsedTime(&ms[rep], e0, e1);
    }
    std::sort(ms.begin(), ms.end());
    const float med = ms[repeats / 2];
    const double bytes = (double)blocks * 4 * ((double)iters + 1) * nl * 1024;
    printf("gather probe: rows %u (%.1f MB), %d waves/CU, %d loads in flight per wave (%d KB per CU), "
           "%.1f%% of row pairs from the whole buffer: median %.3f ms of %d, %.2f TB/s\n",
           rows, rows * 512.0 / 1e6, wpc, nl, wpc * nl, far / 10.0, med, repeats, bytes / (med * 1e-3) / 1e12);
    (void)hipFree(buf);
    (void)hipFree(out);
    return 0;
}
