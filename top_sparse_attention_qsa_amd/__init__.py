"""QSA sparse-attention prefill on MI355X: Python binding of libqsa.so.

The operator (see include/qsa.h) computes, for each query token t and query
head h, softmax(scale * q[t,h] . K_sel^T) V_sel over the token positions the
indexer selected for (t, KV head h // (Hq/Hkv)), masking every slot outside
[0, t] -- "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai, Spanish
page), section "Lo que realmente añade la pull request".

This module only marshals arguments: it checks dtypes, devices and shapes,
makes inputs contiguous, allocates outputs with PyTorch and passes raw device
pointers and the current HIP stream to the C ABI. Every step of the operator
runs in the library's kernels; there is no other implementation to fall back
on, and a missing library is an error.
"""
import ctypes
import math
import os

__all__ = [
    "sparse_prefill",
    "sparse_prefill_extend",
    "sparse_prefill_blocks",
    "sparse_prefill_pool",
    "sparse_decode",
    "sparse_decode_noalloc",
    "decode_workspace_bytes",
    "load_library",
    "library_path",
    "QsaError",
    "STATUS",
    "HEAD_DIM",
]

HEAD_DIM = 256
DEFAULT_SCALE = 1.0 / math.sqrt(HEAD_DIM)
STATUS = {0: "QSA_OK", 1: "QSA_ERR_INVALID_ARG", 2: "QSA_ERR_UNSUPPORTED", 3: "QSA_ERR_LAUNCH"}

_LIB = None


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libqsa.so")


def load_library(path: str = None):
    """Load libqsa.so (built by top_sparse_attention_qsa_amd.build) once.

    `path` selects another build of the same ABI (used to compare kernel
    builds side by side); it replaces the library used by this module."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    path = library_path() if path is None else path
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m top_sparse_attention_qsa_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.qsa_sparse_prefill.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, ctypes.c_float, vp, vp, vp]
    lib.qsa_sparse_prefill.restype = ctypes.c_int
    lib.qsa_sparse_prefill_extend.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32,
                                              ctypes.c_float, vp, vp, vp]
    lib.qsa_sparse_prefill_extend.restype = ctypes.c_int
    lib.qsa_sparse_prefill_blocks.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32,
                                              ctypes.c_float, vp, vp, vp]
    lib.qsa_sparse_prefill_blocks.restype = ctypes.c_int
    lib.qsa_sparse_prefill_pool.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32,
                                            ctypes.c_float, vp, vp, vp]
    lib.qsa_sparse_prefill_pool.restype = ctypes.c_int
    lib.qsa_sparse_decode_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.qsa_sparse_decode_workspace_bytes.restype = i64
    lib.qsa_sparse_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_float, vp, vp,
                                      vp, i64, vp]
    lib.qsa_sparse_decode.restype = ctypes.c_int
    lib.qsa_sparse_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_float, vp,
                                              vp, vp]
    lib.qsa_sparse_decode_noalloc.restype = ctypes.c_int
    lib.qsa_status_string.argtypes = [ctypes.c_int]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_abi_version.argtypes = []
    lib.qsa_abi_version.restype = ctypes.c_int32
    _LIB = lib
    return lib


def _check(status: int, lib) -> None:
    if status != 0:
        raise QsaError(status, lib.qsa_status_string(status).decode())


class _OnDevice:
    """Make device `index` the current HIP device for the call (the library
    launches on the given stream with whatever device is current); no device
    switch at all when it is current already, the common case."""

    __slots__ = ("index", "prev")

    def __init__(self, index):
        self.index = index
        self.prev = None

    def __enter__(self):
        import torch

        cur = torch.cuda.current_device()
        if cur != self.index:
            torch.cuda.set_device(self.index)
            self.prev = cur

    def __exit__(self, *exc):
        if self.prev is not None:
            import torch

            torch.cuda.set_device(self.prev)
        return False


def _on_device(dev):
    return _OnDevice(dev.index)


def _current_stream(dev) -> int:
    """Raw HIP stream handle of the current stream of `dev`."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _prepare(q, k, v, idx, scale, out, lse):
    import torch

    named = (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
             ("v", v, torch.bfloat16), ("idx", idx, torch.int32))
    for name, t, dt in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    for name, t, _ in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
    dev = q.device
    if any(t.device != dev for t in (k, v, idx)):
        raise ValueError("q, k, v and idx must be on the same device")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [T, Hq, {HEAD_DIM}], got {tuple(q.shape)}")
    if k.dim() != 3 or k.shape[2] != HEAD_DIM or v.shape != k.shape:
        raise ValueError(f"k and v must be [T_kv, Hkv, {HEAD_DIM}], got {tuple(k.shape)}, {tuple(v.shape)}")
    T, Hq = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    if idx.dim() != 3 or idx.shape[0] != T or idx.shape[1] != Hkv:
        raise ValueError(f"idx must be [T, Hkv, K] = [{T}, {Hkv}, K], got {tuple(idx.shape)}")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq ({Hq}) must be a positive multiple of Hkv ({Hkv})")
    scale = DEFAULT_SCALE if scale is None else float(scale)
    q, k, v, idx = (t.contiguous() for t in (q, k, v, idx))
    if out is None:
        out = torch.empty((T, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if out.shape != (T, Hq, HEAD_DIM) or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != dev:
        raise ValueError("out must be a contiguous bf16 [T, Hq, 256] tensor on the inputs' device")
    if lse.shape != (T, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev:
        raise ValueError("lse must be a contiguous fp32 [T, Hq] tensor on the inputs' device")
    return q, k, v, idx, scale, out, lse, _current_stream(dev)


def sparse_prefill(q, k, v, idx, scale=None, out=None, lse=None):
    """QSA sparse prefill of one sequence (query row t at position t).

    q [T, Hq, 256] bf16, k/v [T, Hkv, 256] bf16, idx [T, Hkv, K] int32 (-1
    padded, any order), scale defaults to 1/sqrt(256). Returns (out, lse):
    out [T, Hq, 256] bf16, lse [T, Hq] fp32 (natural log; -inf for a row with
    no valid slot, whose out is zero). Runs on the current stream.
    """
    lib = load_library()
    q, k, v, idx, scale, out, lse, stream = _prepare(q, k, v, idx, scale, out, lse)
    if k.shape[0] != q.shape[0]:
        raise ValueError("k and v must have T rows; use sparse_prefill_extend for a longer cache")
    T, Hq, Hkv, K = q.shape[0], q.shape[1], k.shape[1], idx.shape[2]
    with _on_device(q.device):
        st = lib.qsa_sparse_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), T, Hq, Hkv, K,
                                    scale, out.data_ptr(), lse.data_ptr(), stream)
    _check(st, lib)
    return out, lse


def sparse_prefill_extend(q, k, v, idx, q_pos0: int, scale=None, out=None, lse=None):
    """QSA sparse prefill of T new tokens at positions q_pos0 .. q_pos0+T-1
    against a K/V cache of T_kv >= q_pos0 + T rows (slot s valid iff
    0 <= s <= q_pos0 + t)."""
    lib = load_library()
    q, k, v, idx, scale, out, lse, stream = _prepare(q, k, v, idx, scale, out, lse)
    T, Hq, Hkv, K = q.shape[0], q.shape[1], k.shape[1], idx.shape[2]
    with _on_device(q.device):
        st = lib.qsa_sparse_prefill_extend(q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), T,
                                           k.shape[0], int(q_pos0), Hq, Hkv, K, scale, out.data_ptr(),
                                           lse.data_ptr(), stream)
    _check(st, lib)
    return out, lse


def sparse_prefill_blocks(q, k, v, block_idx, q_pos0: int, block_size: int, scale=None, out=None,
                          lse=None):
    """QSA sparse prefill with micro-block indices: entry b of a list names
    tokens b*block_size .. b*block_size+block_size-1 (block_size 1, 2, 4, 8 or
    16), each used iff its position is <= q_pos0 + t. Otherwise as
    sparse_prefill_extend; block_idx is int32 [T, Hkv, n_blocks]."""
    lib = load_library()
    q, k, v, block_idx, scale, out, lse, stream = _prepare(q, k, v, block_idx, scale, out, lse)
    T, Hq, Hkv, nb = q.shape[0], q.shape[1], k.shape[1], block_idx.shape[2]
    with _on_device(q.device):
        st = lib.qsa_sparse_prefill_blocks(q.data_ptr(), k.data_ptr(), v.data_ptr(), block_idx.data_ptr(), T,
                                           k.shape[0], int(q_pos0), Hq, Hkv, nb, int(block_size), scale,
                                           out.data_ptr(), lse.data_ptr(), stream)
    _check(st, lib)
    return out, lse


def _pool_positions(q, k_pool, q_pos, slot_pos):
    import torch

    for name, t, n in (("q_pos", q_pos, q.shape[0]), ("slot_pos", slot_pos, k_pool.shape[0])):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32:
            raise TypeError(f"{name} must be an int32 torch.Tensor")
        if t.device != q.device:
            raise ValueError(f"{name} must be on the inputs' device")
        if t.shape != (n,):
            raise ValueError(f"{name} must have shape ({n},), got {tuple(t.shape)}")
    return q_pos.contiguous(), slot_pos.contiguous()


def sparse_prefill_pool(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, scale=None, out=None, lse=None):
    """QSA sparse prefill of a ragged batch over a shared K/V slot pool.

    q [total_q, Hq, 256] bf16 (rows of all requests concatenated), k_pool /
    v_pool [n_slots, Hkv, 256] bf16, slot_idx [total_q, Hkv, K] int32 pool
    slots, q_pos [total_q] int32 position of each query in its request,
    slot_pos [n_slots] int32 position of the token in each slot (negative:
    empty slot). Slot s is used for row r iff 0 <= s < n_slots and
    0 <= slot_pos[s] <= q_pos[r]."""
    lib = load_library()
    q, k_pool, v_pool, slot_idx, scale, out, lse, stream = _prepare(q, k_pool, v_pool, slot_idx, scale,
                                                                    out, lse)
    q_pos, slot_pos = _pool_positions(q, k_pool, q_pos, slot_pos)
    T, Hq, Hkv, K = q.shape[0], q.shape[1], k_pool.shape[1], slot_idx.shape[2]
    with _on_device(q.device):
        st = lib.qsa_sparse_prefill_pool(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), slot_idx.data_ptr(),
                                         q_pos.data_ptr(), slot_pos.data_ptr(), T, k_pool.shape[0], Hq, Hkv, K,
                                         scale, out.data_ptr(), lse.data_ptr(), stream)
    _check(st, lib)
    return out, lse


def decode_workspace_bytes(n_req: int, Hq: int, Hkv: int, K: int) -> int:
    """Bytes of device workspace sparse_decode needs for these sizes (0: none)."""
    n = load_library().qsa_sparse_decode_workspace_bytes(int(n_req), int(Hq), int(Hkv), int(K))
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def sparse_decode(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, scale=None, out=None, lse=None, workspace=None):
    """One decode step: one query row per request over a K/V slot pool.

    Arguments as sparse_prefill_pool with q [n_req, Hq, 256]. The lists are
    cut into ranges computed in parallel and merged; the partials go to
    `workspace` (a uint8 device tensor of at least decode_workspace_bytes(...)
    bytes, allocated here when None). Calls sharing a workspace must be
    ordered on one stream."""
    import torch

    lib = load_library()
    q, k_pool, v_pool, slot_idx, scale, out, lse, stream = _prepare(q, k_pool, v_pool, slot_idx, scale,
                                                                    out, lse)
    q_pos, slot_pos = _pool_positions(q, k_pool, q_pos, slot_pos)
    n_req, Hq, Hkv, K = q.shape[0], q.shape[1], k_pool.shape[1], slot_idx.shape[2]
    need = decode_workspace_bytes(n_req, Hq, Hkv, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(q.device):
        st = lib.qsa_sparse_decode(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), slot_idx.data_ptr(),
                                   q_pos.data_ptr(), slot_pos.data_ptr(), n_req, k_pool.shape[0], Hq, Hkv, K,
                                   scale, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), ws_bytes, stream)
    _check(st, lib)
    return out, lse


def sparse_decode_noalloc(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, scale=None, out=None, lse=None):
    """sparse_decode with the split partials in the library's own device
    scratch (16 MiB per GPU, held until the process ends) instead of a
    workspace: the library call allocates no memory. Results are bit-identical
    to sparse_decode. Calls that overlap on one GPU (two streams at once) race
    on the scratch; calls on one stream are safe. Pass contiguous inputs and
    `out` and `lse` to keep the whole call free of allocation (this binding
    allocates the outputs, and contiguous copies of strided inputs,
    otherwise)."""
    lib = load_library()
    q, k_pool, v_pool, slot_idx, scale, out, lse, stream = _prepare(q, k_pool, v_pool, slot_idx, scale,
                                                                    out, lse)
    q_pos, slot_pos = _pool_positions(q, k_pool, q_pos, slot_pos)
    n_req, Hq, Hkv, K = q.shape[0], q.shape[1], k_pool.shape[1], slot_idx.shape[2]
    with _on_device(q.device):
        st = lib.qsa_sparse_decode_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                           slot_idx.data_ptr(), q_pos.data_ptr(), slot_pos.data_ptr(), n_req,
                                           k_pool.shape[0], Hq, Hkv, K, scale, out.data_ptr(), lse.data_ptr(),
                                           stream)
    _check(st, lib)
    return out, lse
