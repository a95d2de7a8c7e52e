"""Build the gfx950 shared library libqsa.so in-tree with hipcc.

    python -m top_sparse_attention_qsa_amd.build

Compiles every source under csrc/ (HIP kernels and the C ABI shim) into
top_sparse_attention_qsa_amd/lib/libqsa.so, then the test program
tests/c_driver/qsa_c_driver.cpp (a plain host program that calls the C ABI)
into lib/qsa_c_driver, linked against that library, the gather-ceiling probe
probe/gather_probe.hip (a stand-alone measuring tool) into lib/qsa_gather_probe,
and, with g++, the host
check tests/c_driver/qsa_abi_sanitize.cpp (the ABI's validation under ASan
and UBSan) into lib/qsa_abi_sanitize. Always rebuilds.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libqsa.so")
DRIVER_SRC = os.path.join(ROOT, "tests", "c_driver", "qsa_c_driver.cpp")
DRIVER = os.path.join(LIB_DIR, "qsa_c_driver")
SANITIZE_SRC = os.path.join(ROOT, "tests", "c_driver", "qsa_abi_sanitize.cpp")
SANITIZE = os.path.join(LIB_DIR, "qsa_abi_sanitize")
PROBE_SRC = os.path.join(PKG, "probe", "gather_probe.hip")
PROBE = os.path.join(LIB_DIR, "qsa_gather_probe")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs (the kernels
# rescale them with VALU ops, which cannot address AGPRs).
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqsa.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "is not a recognized feature")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp], verbose)
    os.replace(tmp, LIB)
    if os.path.exists(DRIVER_SRC):
        tmp = DRIVER + ".tmp"
        _run([hipcc(), *HIP_FLAGS, "-I", INCLUDE, DRIVER_SRC, "-L", LIB_DIR, "-lqsa", "-Wl,-rpath,$ORIGIN",
              "-o", tmp], verbose)
        os.replace(tmp, DRIVER)
    if os.path.exists(PROBE_SRC):
        # the gather-ceiling probe: a measuring tool beside the benchmark
        tmp = PROBE + ".tmp"
        _run([hipcc(), *HIP_FLAGS, PROBE_SRC, "-o", tmp], verbose)
        os.replace(tmp, PROBE)
    gxx = shutil.which("g++")
    if os.path.exists(SANITIZE_SRC) and gxx:
        # host code only: the C-ABI validation under ASan/UBSan with a stub launch
        tmp = SANITIZE + ".tmp"
        _run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
              os.path.join(CSRC, "qsa_api.cpp"), SANITIZE_SRC, "-o", tmp], verbose)
        os.replace(tmp, SANITIZE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
