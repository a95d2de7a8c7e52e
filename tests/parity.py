"""Comparison of GPU outputs with the fp64 oracle (helper, not a test module).

Bar: every bf16 output element within 1e-2 of the oracle on top of bf16's own
rounding, i.e. |g - o| <= 1e-2 + ulp_bf16(o) / 2 (the two coincide for
|o| < 2, where almost all outputs lie); every finite lse within 1e-3; empty
rows exactly +0.0 with lse = -inf on both sides.
"""
import numpy as np

OUT_ATOL = 1e-2
LSE_ATOL = 1e-3


def bf16_bits_to_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def half_ulp_bf16(o: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |o| (8 significand bits)."""
    _, ex = np.frexp(np.abs(o))
    return np.ldexp(1.0, np.maximum(ex, -125) - 9)


def torch_bf16_to_numpy_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def compare(out_bits, lse, ref_out, ref_lse, label=""):
    """Assert the bar; return a dict of error statistics."""
    g = bf16_bits_to_f64(out_bits)
    lse = np.asarray(lse, dtype=np.float64)
    assert g.shape == ref_out.shape, (g.shape, ref_out.shape)
    assert lse.shape == ref_lse.shape
    err = np.abs(g - ref_out)
    bound = OUT_ATOL + half_ulp_bf16(ref_out)
    bad = err > bound
    stats = {
        "max_abs_out": float(err.max()) if err.size else 0.0,
        "n_needing_half_ulp": int(np.count_nonzero(err > OUT_ATOL)),
        "rel_l2": float(np.linalg.norm(g - ref_out) / max(np.linalg.norm(ref_out), 1e-300)) if err.size else 0.0,
    }
    fin = np.isfinite(ref_lse)
    if fin.any() and np.array_equal(np.isfinite(lse), fin):
        stats["max_abs_lse"] = float(np.abs(lse[fin] - ref_lse[fin]).max())
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        msg = (f"{label}: {int(bad.sum())} outputs outside the bar; worst at {i}: "
               f"gpu {g[i]!r} oracle {ref_out[i]!r}; {stats}")
        print(msg, flush=True)
        raise AssertionError(msg)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: lse finiteness differs"
    assert np.all(lse[~fin] == ref_lse[~fin]), f"{label}: non-finite lse differs"
    lerr = np.abs(lse[fin] - ref_lse[fin])
    stats["max_abs_lse"] = float(lerr.max()) if lerr.size else 0.0
    assert stats["max_abs_lse"] <= LSE_ATOL, f"{label}: lse error {stats['max_abs_lse']}"
    # empty rows: exactly +0.0 (no negative zero)
    empty = ~fin
    if empty.any():
        ob = np.asarray(out_bits)
        if ob.dtype != np.uint16:
            ob = ob.view(np.uint16)
        assert np.all(ob[empty] == 0), f"{label}: empty rows are not +0.0"
    return stats
