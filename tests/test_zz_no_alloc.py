"""GPU test of the no-allocation decode entry point, qsa_sparse_decode_noalloc.

It runs the same kernels as qsa_sparse_decode with the split partials in the
library's static device scratch instead of a caller's workspace, so its
outputs must equal qsa_sparse_decode's bit for bit, and meet the oracle bar
(tests/parity.py). Calls in a row go through the C ABI (ctypes), each on a
smaller batch than the one before, so each runs over the scratch contents
the previous call left behind; a batch with enough lists that they are not
cut uses no scratch at all. A call captured in a HIP graph replays bit for
bit with other calls in between, through PyTorch's graph capture and from a
plain host program that captures it with the HIP runtime alone.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle
from qsa_inputs import f32_to_bf16_bits, make_pool_inputs
from tests.parity import compare, torch_bf16_to_numpy_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import top_sparse_attention_qsa_amd as qsa  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X: no HIP device visible")
    qsa.load_library()
    return torch.device("cuda", 0)


def progress(msg):
    sys.__stdout__.write(f"    {time.strftime('%H:%M:%S')} {msg}\n")
    sys.__stdout__.flush()


def device_batch(d):
    dev = "cuda"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return bf(d["q"]), bf(d["k"]), bf(d["v"]), i32(d["idx"]), i32(d["q_pos"]), i32(d["slot_pos"])


def both_entry_points(d):
    """(noalloc out, lse), (workspace out, lse) as host arrays, and the bytes
    of scratch the call's split plan uses."""
    args = device_batch(d)
    n, Hq = d["q"].shape[0], d["q"].shape[1]
    out = torch.empty((n, Hq, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, Hq), dtype=torch.float32, device="cuda")
    # stale values in the outputs must not matter either
    out.fill_(3.0)
    lse.fill_(float("nan"))
    o, l = qsa.sparse_decode_noalloc(*args, scale=d["scale"], out=out, lse=lse)
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    ro, rl = qsa.sparse_decode(*args, scale=d["scale"])
    torch.cuda.synchronize()
    need = qsa.decode_workspace_bytes(n, Hq, d["k"].shape[1], d["idx"].shape[2])
    return ((torch_bf16_to_numpy_bits(o), l.cpu().numpy()), (torch_bf16_to_numpy_bits(ro), rl.cpu().numpy()),
            need)


def check_against_decode_and_oracle(d, label):
    (o, l), (ro, rl), need = both_entry_points(d)
    np.testing.assert_array_equal(o, ro, err_msg=label)
    np.testing.assert_array_equal(l.view(np.int32), rl.view(np.int32), err_msg=label)
    ref_out, ref_lse = oracle.sparse_prefill_pool(d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"],
                                                  scale=d["scale"])
    stats = compare(o, l, ref_out, ref_lse, label=label)
    progress(f"{label}: scratch {need} B, identical to qsa_sparse_decode; {stats}")
    return need


def small_batch(seed, n_req, Hq, Hkv, K, n_slots):
    rng = np.random.default_rng(seed)
    f32_to_bf16 = lambda x: f32_to_bf16_bits(x.astype(np.float32))
    slot_pos = rng.permutation(n_slots).astype(np.int32)
    slot_pos[rng.choice(n_slots, n_slots // 10, replace=False)] = -1
    return {
        "q": f32_to_bf16(rng.standard_normal((n_req, Hq, 256))),
        "k": f32_to_bf16(rng.standard_normal((n_slots, Hkv, 256))),
        "v": f32_to_bf16(rng.standard_normal((n_slots, Hkv, 256))),
        "idx": rng.integers(-3, n_slots + 3, size=(n_req, Hkv, K)).astype(np.int32),
        "q_pos": rng.integers(0, n_slots, size=n_req).astype(np.int32),
        "slot_pos": slot_pos,
        "scale": 1 / 16,
    }


def test_noalloc_decode_equals_workspace_decode():
    # first call: the 16-request (24, 2) K = 2,048 decode batch (6.4 MB of scratch)
    big = make_pool_inputs(12)
    need_big = check_against_decode_and_oracle(big, big["cfg"].name)
    # second call, smaller: the 4-request (6, 2) K = 512 batch, over what the first left
    small = make_pool_inputs(11)
    need_small = check_against_decode_and_oracle(small, small["cfg"].name)
    assert 0 < need_small < need_big
    # a third, smaller still, with a different head shape and a 17-slot list
    tiny = small_batch(5, n_req=3, Hq=12, Hkv=1, K=17 * 16 + 5, n_slots=700)
    need_tiny = check_against_decode_and_oracle(tiny, "3 requests (12,1)")
    assert 0 < need_tiny < need_small
    # lists not cut at all (256 lists): no scratch used
    wide = small_batch(6, n_req=256, Hq=4, Hkv=1, K=40, n_slots=900)
    assert check_against_decode_and_oracle(wide, "256 requests, no split") == 0


def test_noalloc_decode_graph_replays():
    """Captured in a HIP graph (the callers this entry point is for) and
    replayed with eager work between replays: each replay equals the eager
    qsa_sparse_decode result bit for bit."""
    d = small_batch(7, n_req=5, Hq=8, Hkv=2, K=700, n_slots=3000)
    args = device_batch(d)
    out = torch.empty((5, 8, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((5, 8), dtype=torch.float32, device="cuda")
    ro, rl = qsa.sparse_decode(*args, scale=d["scale"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside capture (the first call looks up the scratch)
        qsa.sparse_decode_noalloc(*args, scale=d["scale"], out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.sparse_decode_noalloc(*args, scale=d["scale"], out=out, lse=lse)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0.0)
        lse.fill_(0.0)
        other = small_batch(8 + i, n_req=2, Hq=6, Hkv=2, K=300, n_slots=500)  # eager calls in between
        qsa.sparse_decode_noalloc(*device_batch(other), scale=1 / 16)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ro.view(torch.int16)), i
        assert torch.equal(lse.view(torch.int32), rl.view(torch.int32)), i


def test_noalloc_decode_from_a_plain_hip_graph(tmp_path):
    """A plain host program (tests/c_driver/qsa_c_driver.cpp --decode): its
    own hipMalloc buffers and stream, no PyTorch in the process. It makes
    one call, then captures the same call with hipStreamBeginCapture and
    launches the graph twice; the program itself requires every launch to
    reproduce the first call's bits. Its output must also equal the binding's
    qsa_sparse_decode (caller workspace) bit for bit and meet the oracle bar."""
    import subprocess

    from top_sparse_attention_qsa_amd import build as qsa_build

    if not os.path.exists(qsa_build.DRIVER):
        pytest.fail("qsa_c_driver is not built: run __graft_entry__.build() first")
    d = small_batch(9, n_req=3, Hq=12, Hkv=2, K=1500, n_slots=5000)
    n_req, Hq, Hkv, K = 3, 12, 2, 1500
    assert qsa.decode_workspace_bytes(n_req, Hq, Hkv, K) > 0  # the lists are cut: the scratch is used
    (tmp_path / "meta.txt").write_text(f"{n_req} {Hq} {Hkv} {K} {d['k'].shape[0]} {d['scale']}\n")
    for name, key in (("q", "q"), ("k", "k"), ("v", "v"), ("idx", "idx"), ("qpos", "q_pos"), ("spos", "slot_pos")):
        np.ascontiguousarray(d[key]).tofile(tmp_path / f"{name}.bin")
    progress("plain-HIP graph decode: running qsa_c_driver --decode")
    res = subprocess.run([qsa_build.DRIVER, "--decode", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    out_c = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(n_req, Hq, 256)
    lse_c = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(n_req, Hq)
    ro, rl = qsa.sparse_decode(*device_batch(d), scale=d["scale"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_c, torch_bf16_to_numpy_bits(ro))
    np.testing.assert_array_equal(lse_c.view(np.int32), rl.cpu().numpy().view(np.int32))
    ref_out, ref_lse = oracle.sparse_prefill_pool(d["q"], d["k"], d["v"], d["idx"], d["q_pos"], d["slot_pos"],
                                                  scale=d["scale"])
    stats = compare(out_c, lse_c, ref_out, ref_lse, label="plain-HIP graph decode")
    progress(f"plain-HIP graph decode: {res.stdout.strip()}; {stats}")
