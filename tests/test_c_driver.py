"""The C ABI driven by a plain host program (tests/c_driver/qsa_c_driver.cpp):
device buffers from hipMalloc, a HIP stream of its own, no PyTorch and no
Python in the calling process."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from qsa_inputs import f32_to_bf16_bits
from tests.parity import compare, torch_bf16_to_numpy_bits
from top_sparse_attention_qsa_amd import build as qsa_build


def driver() -> str:
    if not os.path.exists(qsa_build.DRIVER):
        pytest.fail("qsa_c_driver is not built: run __graft_entry__.build() first")
    return qsa_build.DRIVER


def test_selftest_runs_without_a_gpu():
    # the ABI version and host-side rejection of invalid arguments: no HIP call is made
    res = subprocess.run([driver(), "--selftest"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "selftest ok" in res.stdout


def test_abi_validation_under_host_sanitizers():
    """The C ABI's argument validation (tests/c_driver/qsa_abi_sanitize.cpp,
    built with g++ -fsanitize=address,undefined and a stub launch) over the
    extremes of every argument and a seeded random mix: no undefined
    behaviour, and every accepted call meets the kernels' preconditions."""
    if not os.path.exists(qsa_build.SANITIZE):
        pytest.fail("qsa_abi_sanitize is not built: run __graft_entry__.build() first")
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0")
    res = subprocess.run([qsa_build.SANITIZE], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 invariant violations" in res.stdout


def ragged_case(seed=2024, T=300, Hq=12, Hkv=2, K=100):
    """T spans several 16-slot tiles with a ragged tail; lists are unordered
    with -1 pads and future positions mixed in."""
    rng = np.random.default_rng(seed)
    bf = lambda shape: f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q, k, v = bf((T, Hq, 256)), bf((T, Hkv, 256)), bf((T, Hkv, 256))
    idx = np.full((T, Hkv, K), -1, np.int32)
    for t in range(T):
        for g in range(Hkv):
            n = min(t + 1, K - 3)
            row = list(rng.choice(t + 1, size=n, replace=False)) + [t + 1 + int(x) for x in rng.integers(0, 9, 2)]
            row += [-1] * (K - len(row))
            rng.shuffle(row)
            idx[t, g] = row
    return q, k, v, idx


@pytest.mark.gpu
def test_plain_host_program_matches_binding_and_oracle(tmp_path):
    import torch

    import top_sparse_attention_qsa_amd as qsa

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: no HIP device visible")
    q, k, v, idx = ragged_case()
    T, Hq, Hkv, K = q.shape[0], q.shape[1], k.shape[1], idx.shape[2]
    (tmp_path / "meta.txt").write_text(f"{T} {Hq} {Hkv} {K} 0.0625\n")
    for name, a in (("q", q), ("k", k), ("v", v), ("idx", idx)):
        np.ascontiguousarray(a).tofile(tmp_path / f"{name}.bin")
    res = subprocess.run([driver(), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    out_c = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(T, Hq, 256)
    lse_c = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(T, Hq)

    # the same call through the Python binding: the same kernel, so the same bits
    bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to("cuda")
    out_p, lse_p = qsa.sparse_prefill(bf16(q), bf16(k), bf16(v), torch.from_numpy(idx).to("cuda"), scale=0.0625)
    torch.cuda.synchronize()
    assert np.array_equal(out_c, torch_bf16_to_numpy_bits(out_p))
    assert np.array_equal(lse_c.view(np.uint32), lse_p.cpu().numpy().view(np.uint32))

    ref_out, ref_lse = oracle.sparse_prefill(q, k, v, idx, scale=0.0625)
    compare(out_c, lse_c, ref_out, ref_lse, label="c driver")


def test_gather_probe_rejects_bad_arguments():
    """The gather-ceiling probe (a measuring tool built beside the library)
    checks its arguments before any HIP call: buffer size, waves per CU and
    loads in flight outside their ranges are refused with status 2."""
    probe = qsa_build.PROBE
    if not os.path.exists(probe):
        pytest.fail("qsa_gather_probe is not built: run __graft_entry__.build() first")
    for args in ([], ["8192", "8", "100"], ["1", "8", "100", "16"], ["4194304", "8", "100", "16"],
                 ["8192", "6", "100", "16"], ["8192", "8", "0", "16"], ["8192", "8", "100", "12"],
                 ["8192", "8", "100", "16", "0"], ["8192", "8", "100", "16", "5", "1001"]):
        res = subprocess.run([probe, *args], capture_output=True, text=True, timeout=60)
        assert res.returncode == 2, (args, res.stderr)
