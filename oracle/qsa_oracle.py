"""Plain fp64 CPU oracle for the QSA sparse-prefill operator.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the package
entry point and the CPU-baseline leg of the benchmark use it. It shares no
code, header, table or helper with the HIP kernels, and it imports nothing
from the GPU package or from the input generators.

What it computes -- "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai,
Spanish page), section "Lo que realmente añade la pull request": for already
rotated Q and K, attention over the indexer-selected tokens is
softmax(scale * Q K_sel^T) V_sel, with the original head-dim-256 scale kept
(1/sqrt(256)); index slots holding -1 are masked, and a row left with no
selected token keeps the convention of a zero output. Section "Nueve pruebas
que pasaron" adds the test facts this follows: unordered physical slots,
default and explicit scales, fully masked rows, zero selection width, causal
tails. The operator is causal: a query at position t only sees positions
s <= t.

Readings taken where the pages leave a step open:
  * query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous GQA
    groups; the pages batch per KV head and pad heads inside each group);
  * a slot s is used iff 0 <= s <= t; every other value (-1, any negative,
    a future position, s >= T) is masked, not an error;
  * each list entry is one softmax term, so a repeated position counts as
    many times as it appears (parity unpinned for repeats: the workloads
    never repeat a position);
  * an empty row gives out = +0.0 and lse = -inf (log of an empty sum);
  * lse is the natural log of sum_j exp(scale * q . k_j).

Arithmetic is float64 throughout; bf16 inputs widen to float64 exactly.
"""
import numpy as np

D = 256


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64.

    A bf16 value is the top half of the float32 with the same bits, so the
    widening is a 16-bit shift followed by an exact float32 -> float64 cast.
    Float arrays are passed through as float64.
    """
    a = np.asarray(bits)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def kv_head_of(h: int, G: int) -> int:
    """KV head read by query head h: contiguous groups of G query heads."""
    return h // G


def selected_positions(idx_row, t: int) -> list:
    """The positions a query at position t attends to: the entries s of its
    index list with 0 <= s <= t, in list order (repeats kept)."""
    return [int(s) for s in idx_row if 0 <= int(s) <= t]


def attend(q_h: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float):
    """softmax(scale * q . k_j) weighted sum of v_j for one query head.

    Returns (out[D], lse, p[n]) in float64. With no selected key: out = +0.0,
    lse = -inf, p empty.
    """
    n = k_sel.shape[0]
    if n == 0:
        return np.zeros(q_h.shape[-1]), -np.inf, np.zeros(0)
    z = scale * (k_sel @ q_h)  # logits, one per selected key
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    p = w / l
    out = p @ v_sel
    return out, m + np.log(l), p


def sparse_prefill(q, k, v, idx, scale: float = None, rows=None, Hq: int = None, Hkv: int = None,
                   q_pos0: int = 0):
    """Reference outputs of the QSA sparse-prefill operator.

    q    [T, Hq, 256]     bf16 bits (uint16) or floats
    k, v [T_kv, Hkv, 256] bf16 bits (uint16) or floats
    idx  [T, Hkv, K]      int token positions (or [len(rows), Hkv, K] when
                          `rows` is given and idx holds only those rows)
    rows   optional query rows to evaluate (default: all T rows)
    q_pos0 absolute position of query row 0 (tokens already in the cache);
           query row t attends to positions 0 <= s <= q_pos0 + t

    Returns out float64 [R, Hq, 256] and lse float64 [R, Hq].
    """
    q = np.asarray(q)
    T = q.shape[0]
    Hq = q.shape[1] if Hq is None else Hq
    Hkv = np.asarray(k).shape[1] if Hkv is None else Hkv
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    idx = np.asarray(idx)
    if rows is None:
        rows = np.arange(T)
        idx_rows = idx
    else:
        rows = np.asarray(rows, dtype=np.int64)
        idx_rows = idx if idx.shape[0] == rows.size else idx[rows]
    k = np.asarray(k)
    v = np.asarray(v)
    out = np.zeros((rows.size, Hq, D))
    lse = np.full((rows.size, Hq), -np.inf)
    for i, t in enumerate(rows):
        q_t = bf16_to_f64(q[t])
        for g in range(Hkv):
            sel = selected_positions(idx_rows[i, g], int(q_pos0) + int(t))
            k_sel = bf16_to_f64(k[sel, g, :]) if sel else np.zeros((0, D))
            v_sel = bf16_to_f64(v[sel, g, :]) if sel else np.zeros((0, D))
            for h in range(Hq):
                if kv_head_of(h, G) != g:
                    continue
                o, l, _ = attend(q_t[h], k_sel, v_sel, scale)
                out[i, h] = o
                lse[i, h] = l
    return out, lse


def row_probabilities(q, k, idx, t: int, h: int, scale: float = None, Hkv: int = None):
    """Selected positions and softmax weights of query head h at row t
    (for probability-level checks)."""
    q = np.asarray(q)
    Hq = q.shape[1]
    Hkv = np.asarray(k).shape[1] if Hkv is None else Hkv
    G = Hq // Hkv
    g = kv_head_of(h, G)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    sel = selected_positions(np.asarray(idx)[t, g], t)
    k_sel = bf16_to_f64(np.asarray(k)[sel, g, :]) if sel else np.zeros((0, D))
    q_h = bf16_to_f64(q[t, h])
    n = len(sel)
    z = scale * (k_sel @ q_h) if n else np.zeros(0)
    _, lse, p = attend(q_h, k_sel, np.zeros((n, D)), scale)
    return sel, z, p, lse
