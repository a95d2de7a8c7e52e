"""The C ABI library: it loads, exports every entry point include/qsa.h
declares, and rejects invalid arguments on the host before any HIP call
(no GPU needed: every call here returns before touching a device)."""
import ctypes
import os
import re

import pytest

import top_sparse_attention_qsa_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

OK, INVALID, UNSUPPORTED, LAUNCH = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qsa.library_path()):
        pytest.fail("libqsa.so is not built: run __graft_entry__.build() first")
    return qsa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(qsa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == ["qsa_abi_version", "qsa_sparse_decode", "qsa_sparse_decode_noalloc",
                     "qsa_sparse_decode_workspace_bytes",
                     "qsa_sparse_prefill", "qsa_sparse_prefill_blocks", "qsa_sparse_prefill_extend",
                     "qsa_sparse_prefill_pool", "qsa_status_string"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libqsa.so does not export {name}"


def test_abi_version_and_status_strings(lib):
    assert lib.qsa_abi_version() == 3
    assert lib.qsa_status_string(OK) == b"ok"
    assert lib.qsa_status_string(INVALID) == b"invalid argument"
    assert lib.qsa_status_string(UNSUPPORTED) == b"unsupported size"
    assert lib.qsa_status_string(LAUNCH) == b"kernel launch failed"
    assert lib.qsa_status_string(99) == b"unknown status"


# Distinct non-null host addresses stand in for device pointers: validation
# rejects the call before any of them is used.
P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(7)]
Q, K_, V, IDX, OUT, LSE, STREAM = P


def call(lib, q=Q, k=K_, v=V, idx=IDX, T=8, Hq=4, Hkv=2, K=5, scale=0.0625, out=OUT, lse=LSE):
    return lib.qsa_sparse_prefill(q, k, v, idx, T, Hq, Hkv, K, scale, out, lse, None)


def call_ext(lib, T=8, T_kv=20, p0=4, Hq=4, Hkv=2, K=5, scale=0.0625, q=Q, out=OUT):
    return lib.qsa_sparse_prefill_extend(q, K_, V, IDX, T, T_kv, p0, Hq, Hkv, K, scale, out, LSE, None)


@pytest.mark.parametrize("kwargs", [
    dict(T=-1), dict(T=2 ** 31), dict(Hq=0), dict(Hkv=0), dict(Hq=-3), dict(K=-1),
    dict(Hq=6, Hkv=4), dict(Hq=3, Hkv=2), dict(scale=float("nan")), dict(scale=float("inf")),
    dict(scale=float("-inf")), dict(q=None), dict(out=None), dict(lse=None), dict(k=None),
    dict(v=None), dict(idx=None), dict(out=Q), dict(out=K_), dict(lse=IDX), dict(lse=OUT),
])
def test_invalid_arguments_are_rejected(lib, kwargs):
    assert call(lib, **kwargs) == INVALID


def test_unsupported_sizes(lib):
    # T * Hkv * 512 bytes of K must stay below 2^31
    assert call(lib, T=4194304, Hq=1, Hkv=1) == UNSUPPORTED
    assert call(lib, T=2097152, Hq=4, Hkv=2) == UNSUPPORTED
    assert call(lib, K=(1 << 28) + 1) == UNSUPPORTED


def test_zero_tokens_is_a_noop(lib):
    assert call(lib, T=0) == OK
    assert call(lib, T=0, q=None, k=None, v=None, idx=None, out=None, lse=None) == OK


def test_null_index_rejected_only_when_used(lib):
    # K == 0: idx, k and v are never read; with T == 0 nothing is launched either
    assert call(lib, T=0, K=0, idx=None) == OK


@pytest.mark.parametrize("kwargs,expect", [
    (dict(p0=-1), INVALID), (dict(T=8, T_kv=11, p0=4), INVALID), (dict(T_kv=-2), INVALID),
    (dict(T=0, T_kv=0, p0=0), OK), (dict(T=0, T_kv=100, p0=100), OK),
    (dict(T=8, T_kv=4194304, p0=0, Hkv=1, Hq=1), UNSUPPORTED),
    # query positions past the cache, also where q_pos0 + T would overflow int64
    (dict(T=5, T_kv=10, p0=2 ** 63 - 2), INVALID), (dict(T=2 ** 62, T_kv=2 ** 62, p0=2 ** 62), INVALID),
    (dict(T=1, T_kv=2 ** 62, p0=2 ** 62), INVALID),
])
def test_extend_argument_rules(lib, kwargs, expect):
    assert call_ext(lib, **kwargs) == expect


def call_blk(lib, T=8, T_kv=20, p0=4, Hq=4, Hkv=2, nb=5, bs=4, scale=0.0625, idx=IDX):
    return lib.qsa_sparse_prefill_blocks(Q, K_, V, idx, T, T_kv, p0, Hq, Hkv, nb, bs, scale, OUT, LSE, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(bs=0), INVALID), (dict(bs=3), INVALID), (dict(bs=32), INVALID), (dict(bs=-4), INVALID),
    (dict(nb=-1), INVALID), (dict(p0=-1), INVALID), (dict(T=8, T_kv=11, p0=4), INVALID),
    (dict(idx=None), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(nb=(1 << 26) + 1, bs=4), UNSUPPORTED), (dict(nb=(1 << 24) + 1, bs=16), UNSUPPORTED),
    (dict(T=0, nb=1 << 24, bs=16), OK), (dict(T=0, bs=16), OK), (dict(T=0, bs=5), INVALID),
])
def test_blocks_argument_rules(lib, kwargs, expect):
    assert call_blk(lib, **kwargs) == expect


QP, SP = ctypes.c_void_p(0x90000), ctypes.c_void_p(0xA0000)


def call_pool(lib, total_q=8, n_slots=40, Hq=4, Hkv=2, K=5, scale=0.0625, q_pos=QP, slot_pos=SP, out=OUT,
              lse=LSE, idx=IDX):
    return lib.qsa_sparse_prefill_pool(Q, K_, V, idx, q_pos, slot_pos, total_q, n_slots, Hq, Hkv, K, scale,
                                       out, lse, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(total_q=-1), INVALID), (dict(n_slots=-1), INVALID), (dict(total_q=2 ** 31), INVALID),
    (dict(n_slots=2 ** 31), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(K=-2), INVALID),
    (dict(q_pos=None), INVALID), (dict(slot_pos=None), INVALID), (dict(idx=None), INVALID),
    (dict(out=QP), INVALID), (dict(lse=SP), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(n_slots=4194304, Hkv=1, Hq=1), UNSUPPORTED), (dict(K=(1 << 28) + 1), UNSUPPORTED),
    (dict(total_q=0), OK), (dict(total_q=0, q_pos=None, slot_pos=None), OK),
    (dict(n_slots=0, q_pos=None), INVALID), (dict(n_slots=0, idx=None), INVALID),
])
def test_pool_argument_rules(lib, kwargs, expect):
    assert call_pool(lib, **kwargs) == expect


def test_python_binding_validates_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(4, 2, 256, dtype=torch.bfloat16)
    k = torch.zeros(4, 1, 256, dtype=torch.bfloat16)
    idx = torch.zeros(4, 1, 3, dtype=torch.int32)
    with pytest.raises(ValueError):  # host tensors are refused
        qsa.sparse_prefill(q, k, k, idx)
    with pytest.raises(TypeError):
        qsa.sparse_prefill(q.float(), k, k, idx)
    with pytest.raises(TypeError):
        qsa.sparse_prefill(q, k, k, idx.long())


WS = ctypes.c_void_p(0xB0000)


def call_dec(lib, n_req=16, n_slots=1000, Hq=24, Hkv=2, K=2048, scale=0.0625, q_pos=QP, slot_pos=SP, out=OUT,
             lse=LSE, idx=IDX, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = max(lib.qsa_sparse_decode_workspace_bytes(n_req, Hq, Hkv, K), 0)
    return lib.qsa_sparse_decode(Q, K_, V, idx, q_pos, slot_pos, n_req, n_slots, Hq, Hkv, K, scale, out, lse,
                                 ws, ws_bytes, None)


def test_decode_workspace_sizes(lib):
    f = lib.qsa_sparse_decode_workspace_bytes
    # 16 requests x 2 KV heads = 32 lists of 128 tiles, cut into 16 ranges of
    # 8 tiles: (16 * 24 heads * 16 ranges) records of 16 + 1024 bytes
    assert f(16, 24, 2, 2048) == 16 * 24 * 16 * 1040
    assert f(1, 24, 2, 2048) == 24 * 128 * 1040  # one tile per range
    assert f(128, 24, 2, 2048) == 0               # 256 lists: no cut
    assert f(127, 24, 2, 2048) == 127 * 24 * 2 * 1040
    assert f(4, 6, 2, 16) == 0                    # one tile: nothing to cut
    assert f(0, 24, 2, 2048) == 0
    for bad in [(-1, 24, 2, 8), (2 ** 31, 24, 2, 8), (4, 0, 2, 8), (4, 6, 4, 8), (4, 6, 2, -1), (4, 6, 2, (1 << 28) + 1)]:
        assert f(*bad) == -1


@pytest.mark.parametrize("kwargs,expect", [
    (dict(n_req=-1), INVALID), (dict(q_pos=None), INVALID), (dict(slot_pos=None), INVALID),
    (dict(ws=None), INVALID), (dict(ws_bytes=100), INVALID), (dict(ws_bytes=-1), INVALID),
    (dict(ws=ctypes.c_void_p(0xB0008)), INVALID), (dict(ws=QP), INVALID), (dict(ws=Q), INVALID),
    (dict(ws=OUT), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(n_slots=4194304, Hkv=1, Hq=1), UNSUPPORTED), (dict(n_req=0), OK),
    (dict(n_req=0, q_pos=None, slot_pos=None, ws=None), OK),
])
def test_decode_argument_rules(lib, kwargs, expect):
    assert call_dec(lib, **kwargs) == expect


DECODE_SCRATCH_BYTES = 16 << 20  # QSA_DECODE_SCRATCH_BYTES in include/qsa.h


def test_header_states_the_scratch_size():
    assert re.search(r"#define QSA_DECODE_SCRATCH_BYTES \(16LL << 20\)", open(HEADER).read())


def test_every_decode_plan_fits_the_static_scratch(lib):
    """The no-allocation decode keeps its partials in a 16 MiB scratch: the
    workspace of every split plan fits it (the bound is 16 * 767 rows of
    1,040 bytes), over request counts up to the no-split limit, head groups
    of 1..48 (several 16-head chunks included) and list widths up to 2^28."""
    f = lib.qsa_sparse_decode_workspace_bytes
    worst = 0
    for n_req in list(range(1, 40)) + [63, 64, 85, 100, 127, 128, 200, 255, 256, 300]:
        for Hkv in (1, 2, 3, 4, 8):
            for G in (1, 3, 6, 8, 12, 16, 17, 24, 32, 48):
                for K in (17, 64, 2048, 2051, 65536, 1 << 20, 1 << 28):
                    need = f(n_req, Hkv * G, Hkv, K)
                    assert 0 <= need <= DECODE_SCRATCH_BYTES, (n_req, Hkv, G, K, need)
                    worst = max(worst, need)
    assert worst > DECODE_SCRATCH_BYTES // 2  # the sweep reaches near the bound


def call_noalloc(lib, n_req=16, n_slots=1000, Hq=24, Hkv=2, K=2048, scale=0.0625, q_pos=QP, slot_pos=SP, out=OUT,
                 lse=LSE, idx=IDX, q=Q):
    return lib.qsa_sparse_decode_noalloc(q, K_, V, idx, q_pos, slot_pos, n_req, n_slots, Hq, Hkv, K, scale, out,
                                         lse, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(n_req=-1), INVALID), (dict(n_req=2 ** 31), INVALID), (dict(q_pos=None), INVALID),
    (dict(slot_pos=None), INVALID), (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(lse=None), INVALID),
    (dict(idx=None), INVALID), (dict(out=QP), INVALID), (dict(lse=SP), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(Hq=0), INVALID), (dict(K=-1), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(n_slots=4194304, Hkv=1, Hq=1), UNSUPPORTED), (dict(K=(1 << 28) + 1), UNSUPPORTED),
    (dict(n_req=0), OK), (dict(n_req=0, q_pos=None, slot_pos=None), OK),
])
def test_decode_noalloc_argument_rules(lib, kwargs, expect):
    """The no-allocation decode validates like qsa_sparse_decode, on the
    host, before its first HIP call (none of these calls reaches a device)."""
    assert call_noalloc(lib, **kwargs) == expect
