// A plain host program that calls the QSA C ABI (include/qsa.h) with buffers
// from hipMalloc and a stream of its own: no PyTorch, no Python.
//
//   qsa_c_driver <dir>      reads <dir>/meta.txt ("T Hq Hkv K scale"),
//                           q.bin / k.bin / v.bin (bf16 bits, row-major
//                           [T,Hq,256] / [T,Hkv,256]) and idx.bin (int32
//                           [T,Hkv,K]); runs qsa_sparse_prefill; writes
//                           out.bin (bf16 bits [T,Hq,256]) and lse.bin
//                           (fp32 [T,Hq]).
//   qsa_c_driver --decode <dir>
//                           reads <dir>/meta.txt ("n_req Hq Hkv K n_slots
//                           scale"), q.bin ([n_req,Hq,256] bf16 bits),
//                           k.bin / v.bin ([n_slots,Hkv,256]), idx.bin (int32
//                           [n_req,Hkv,K]), qpos.bin (int32 [n_req]) and
//                           spos.bin (int32 [n_slots]); runs
//                           qsa_sparse_decode_noalloc once on its stream,
//                           then captures the same call in a HIP graph
//                           (hipStreamBeginCapture), instantiates it and
//                           launches it twice, the outputs overwritten in
//                           between; every launch must reproduce the first
//                           call's bits. Writes out.bin and lse.bin.
//   qsa_c_driver --selftest checks the ABI version and that invalid
//                           arguments are refused before any HIP call
//                           (runs without a GPU).
//
// Exit status 0 on success; any failure prints a message and exits 1.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qsa.h"

namespace {

bool fail(const char *what) {
    std::fprintf(stderr, "qsa_c_driver: %s\n", what);
    return false;
}

bool hip_ok(hipError_t e, const char *what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "qsa_c_driver: %s: %s\n", what, hipGetErrorString(e));
    return false;
}

template <typename T>
bool read_file(const std::string &path, std::vector<T> &buf, size_t count) {
    buf.resize(count);
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f) return fail(("cannot open " + path).c_str());
    const size_t got = count ? std::fread(buf.data(), sizeof(T), count, f) : 0;
    std::fclose(f);
    if (got != count) return fail(("short read of " + path).c_str());
    return true;
}

template <typename T>
bool write_file(const std::string &path, const std::vector<T> &buf) {
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f) return fail(("cannot create " + path).c_str());
    const size_t put = buf.empty() ? 0 : std::fwrite(buf.data(), sizeof(T), buf.size(), f);
    std::fclose(f);
    if (put != buf.size()) return fail(("short write of " + path).c_str());
    return true;
}

int selftest() {
    if (qsa_abi_version() != QSA_ABI_VERSION) return fail("ABI version mismatch"), 1;
    // Hq not a multiple of Hkv: refused on the host; the pointers are never read
    static uint16_t dummy[256];
    static int32_t idx[1];
    static float lse[3];
    const qsa_status_t st = qsa_sparse_prefill(dummy, dummy, dummy, idx, 1, 3, 2, 1, 0.0625f, dummy + 8, lse,
                                               nullptr);
    if (st != QSA_ERR_INVALID_ARG) return fail("Hq % Hkv != 0 was not refused"), 1;
    // T == 0 is a no-op with any pointers
    if (qsa_sparse_prefill(nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 8, 0.0625f, nullptr, nullptr, nullptr) !=
        QSA_OK)
        return fail("T == 0 was not a no-op"), 1;
    std::printf("selftest ok: abi %d, invalid args -> \"%s\"\n", qsa_abi_version(), qsa_status_string(st));
    return 0;
}

int run(const std::string &dir) {
    long long T = 0;
    int Hq = 0, Hkv = 0, K = 0;
    float scale = 0.f;
    {
        FILE *f = std::fopen((dir + "/meta.txt").c_str(), "r");
        if (!f) return fail("cannot open meta.txt"), 1;
        const int n = std::fscanf(f, "%lld %d %d %d %f", &T, &Hq, &Hkv, &K, &scale);
        std::fclose(f);
        if (n != 5 || T < 1 || Hq < 1 || Hkv < 1 || K < 0) return fail("bad meta.txt"), 1;
    }
    const size_t nq = (size_t)T * Hq * 256, nkv = (size_t)T * Hkv * 256, ni = (size_t)T * Hkv * K;
    std::vector<uint16_t> q, k, v, out(nq);
    std::vector<int32_t> idx;
    std::vector<float> lse((size_t)T * Hq);
    if (!read_file(dir + "/q.bin", q, nq) || !read_file(dir + "/k.bin", k, nkv) ||
        !read_file(dir + "/v.bin", v, nkv) || !read_file(dir + "/idx.bin", idx, ni))
        return 1;

    hipStream_t stream = nullptr;
    void *dq = nullptr, *dk = nullptr, *dv = nullptr, *di = nullptr, *dout = nullptr, *dlse = nullptr;
    bool ok = hip_ok(hipStreamCreate(&stream), "hipStreamCreate") &&
              hip_ok(hipMalloc(&dq, nq * 2), "hipMalloc q") && hip_ok(hipMalloc(&dk, nkv * 2), "hipMalloc k") &&
              hip_ok(hipMalloc(&dv, nkv * 2), "hipMalloc v") &&
              hip_ok(hipMalloc(&di, ni * 4 + 4), "hipMalloc idx") &&
              hip_ok(hipMalloc(&dout, nq * 2), "hipMalloc out") &&
              hip_ok(hipMalloc(&dlse, lse.size() * 4), "hipMalloc lse") &&
              hip_ok(hipMemcpyAsync(dq, q.data(), nq * 2, hipMemcpyHostToDevice, stream), "copy q") &&
              hip_ok(hipMemcpyAsync(dk, k.data(), nkv * 2, hipMemcpyHostToDevice, stream), "copy k") &&
              hip_ok(hipMemcpyAsync(dv, v.data(), nkv * 2, hipMemcpyHostToDevice, stream), "copy v") &&
              (ni == 0 || hip_ok(hipMemcpyAsync(di, idx.data(), ni * 4, hipMemcpyHostToDevice, stream), "copy idx"));
    if (ok) {
        const qsa_status_t st = qsa_sparse_prefill(dq, dk, dv, (const int32_t *)di, T, Hq, Hkv, K, scale, dout,
                                                   (float *)dlse, stream);
        if (st != QSA_OK) {
            std::fprintf(stderr, "qsa_c_driver: qsa_sparse_prefill: %s\n", qsa_status_string(st));
            ok = false;
        }
    }
    ok = ok && hip_ok(hipMemcpyAsync(out.data(), dout, nq * 2, hipMemcpyDeviceToHost, stream), "copy out") &&
         hip_ok(hipMemcpyAsync(lse.data(), dlse, lse.size() * 4, hipMemcpyDeviceToHost, stream), "copy lse") &&
         hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize");
    for (void *p : {dq, dk, dv, di, dout, dlse})
        if (p) (void)hipFree(p);
    if (stream) (void)hipStreamDestroy(stream);
    if (!ok || !write_file(dir + "/out.bin", out) || !write_file(dir + "/lse.bin", lse)) return 1;
    std::printf("ok: T=%lld Hq=%d Hkv=%d K=%d\n", T, Hq, Hkv, K);
    return 0;
}

// One decode step through the no-allocation entry point: a plain call, then
// the same call replayed from a HIP graph captured on the caller's stream.
int run_decode(const std::string &dir) {
    long long n_req = 0, n_slots = 0;
    int Hq = 0, Hkv = 0, K = 0;
    float scale = 0.f;
    {
        FILE *f = std::fopen((dir + "/meta.txt").c_str(), "r");
        if (!f) return fail("cannot open meta.txt"), 1;
        const int n = std::fscanf(f, "%lld %d %d %d %lld %f", &n_req, &Hq, &Hkv, &K, &n_slots, &scale);
        std::fclose(f);
        if (n != 6 || n_req < 1 || n_req > 4096 || Hq < 1 || Hkv < 1 || K < 1 || K > (1 << 20) || n_slots < 1 ||
            n_slots > (1 << 22))
            return fail("bad meta.txt"), 1;
    }
    const size_t nq = (size_t)n_req * Hq * 256, nkv = (size_t)n_slots * Hkv * 256;
    const size_t ni = (size_t)n_req * Hkv * K, nl = (size_t)n_req * Hq;
    std::vector<uint16_t> q, k, v, out(nq), out0(nq);
    std::vector<int32_t> idx, qpos, spos;
    std::vector<float> lse(nl), lse0(nl);
    if (!read_file(dir + "/q.bin", q, nq) || !read_file(dir + "/k.bin", k, nkv) ||
        !read_file(dir + "/v.bin", v, nkv) || !read_file(dir + "/idx.bin", idx, ni) ||
        !read_file(dir + "/qpos.bin", qpos, (size_t)n_req) || !read_file(dir + "/spos.bin", spos, (size_t)n_slots))
        return 1;

    hipStream_t stream = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    void *dq = nullptr, *dk = nullptr, *dv = nullptr, *di = nullptr, *dqp = nullptr, *dsp = nullptr;
    void *dout = nullptr, *dlse = nullptr;
    auto call = [&]() -> bool {
        const qsa_status_t st = qsa_sparse_decode_noalloc(dq, dk, dv, (const int32_t *)di, (const int32_t *)dqp,
                                                          (const int32_t *)dsp, n_req, n_slots, Hq, Hkv, K, scale,
                                                          dout, (float *)dlse, stream);
        if (st == QSA_OK) return true;
        std::fprintf(stderr, "qsa_c_driver: qsa_sparse_decode_noalloc: %s\n", qsa_status_string(st));
        return false;
    };
    auto fetch = [&](std::vector<uint16_t> &o, std::vector<float> &l) -> bool {
        return hip_ok(hipMemcpyAsync(o.data(), dout, nq * 2, hipMemcpyDeviceToHost, stream), "copy out") &&
               hip_ok(hipMemcpyAsync(l.data(), dlse, nl * 4, hipMemcpyDeviceToHost, stream), "copy lse") &&
               hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize");
    };
    // overwrite the outputs, so that a launch that wrote nothing cannot pass
    auto scrub = [&]() -> bool {
        return hip_ok(hipMemsetAsync(dout, 0x7F, nq * 2, stream), "scrub out") &&
               hip_ok(hipMemsetAsync(dlse, 0x7F, nl * 4, stream), "scrub lse");
    };
    bool ok = hip_ok(hipStreamCreate(&stream), "hipStreamCreate") && hip_ok(hipMalloc(&dq, nq * 2), "hipMalloc q") &&
              hip_ok(hipMalloc(&dk, nkv * 2), "hipMalloc k") && hip_ok(hipMalloc(&dv, nkv * 2), "hipMalloc v") &&
              hip_ok(hipMalloc(&di, ni * 4), "hipMalloc idx") && hip_ok(hipMalloc(&dqp, n_req * 4), "hipMalloc q_pos") &&
              hip_ok(hipMalloc(&dsp, n_slots * 4), "hipMalloc slot_pos") &&
              hip_ok(hipMalloc(&dout, nq * 2), "hipMalloc out") && hip_ok(hipMalloc(&dlse, nl * 4), "hipMalloc lse") &&
              hip_ok(hipMemcpyAsync(dq, q.data(), nq * 2, hipMemcpyHostToDevice, stream), "copy q") &&
              hip_ok(hipMemcpyAsync(dk, k.data(), nkv * 2, hipMemcpyHostToDevice, stream), "copy k") &&
              hip_ok(hipMemcpyAsync(dv, v.data(), nkv * 2, hipMemcpyHostToDevice, stream), "copy v") &&
              hip_ok(hipMemcpyAsync(di, idx.data(), ni * 4, hipMemcpyHostToDevice, stream), "copy idx") &&
              hip_ok(hipMemcpyAsync(dqp, qpos.data(), n_req * 4, hipMemcpyHostToDevice, stream), "copy q_pos") &&
              hip_ok(hipMemcpyAsync(dsp, spos.data(), n_slots * 4, hipMemcpyHostToDevice, stream), "copy slot_pos");
    // the plain call first (on a device, the first call looks up the scratch)
    ok = ok && scrub() && call() && fetch(out0, lse0);
    // the same call captured in a graph: no allocation happens inside it
    if (ok) {
        ok = hip_ok(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal), "hipStreamBeginCapture");
        const bool called = ok && call();
        hipGraph_t g = nullptr;
        const bool ended = ok && hip_ok(hipStreamEndCapture(stream, &g), "hipStreamEndCapture");
        graph = g;
        ok = called && ended && hip_ok(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "hipGraphInstantiate");
    }
    for (int rep = 0; ok && rep < 2; ++rep) {
        ok = scrub() && hip_ok(hipGraphLaunch(exec, stream), "hipGraphLaunch") && fetch(out, lse);
        if (ok && (out != out0 || std::memcmp(lse.data(), lse0.data(), nl * 4) != 0)) {
            std::fprintf(stderr, "qsa_c_driver: graph launch %d differs from the plain call\n", rep);
            ok = false;
        }
    }
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    for (void *p : {dq, dk, dv, di, dqp, dsp, dout, dlse})
        if (p) (void)hipFree(p);
    if (stream) (void)hipStreamDestroy(stream);
    if (!ok || !write_file(dir + "/out.bin", out) || !write_file(dir + "/lse.bin", lse)) return 1;
    std::printf("ok: decode n_req=%lld Hq=%d Hkv=%d K=%d n_slots=%lld, 2 graph launches equal the plain call\n", n_req,
                Hq, Hkv, K, n_slots);
    return 0;
}

} // namespace

int main(int argc, char **argv) {
    if (argc == 2 && std::string(argv[1]) == "--selftest") return selftest();
    if (argc == 3 && std::string(argv[1]) == "--decode") return run_decode(argv[2]);
    if (argc != 2) {
        std::fprintf(stderr, "usage: qsa_c_driver <dir> | --decode <dir> | --selftest\n");
        return 1;
    }
    return run(argv[1]);
}
