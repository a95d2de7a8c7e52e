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

Two further forms of the same operation (same section "Nueve pruebas que
pasaron", and section "Por qué QSA es la parte incómoda, en cifras" for the
model's micro-blocks):
  * micro-block indices: the model's indexer selects micro-blocks at a
    compression ratio of 4; an entry b names tokens b*B .. b*B+B-1 in that
    order, and each of them is causal-masked on its own, so the block that
    holds the query keeps only its first (t mod B) + 1 tokens;
  * a batch of requests over one pool of physical K/V slots (two requests may
    share the slots of a common prefix): an entry is a slot number, the slot
    records the position of the token it holds (negative: an empty slot), and
    the slot is used iff it exists, holds a token, and that token's position
    is <= the query's position in its own request.

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


def expand_blocks(block_row, block_size: int) -> list:
    """Token positions named by a list of micro-block entries, in list order:
    entry b names b*block_size, b*block_size + 1, ..., b*block_size +
    block_size - 1. Nothing is dropped here; causality and range are applied
    per token afterwards, exactly as for token lists."""
    return [int(b) * block_size + i for b in block_row for i in range(block_size)]


def sparse_prefill_blocks(q, k, v, block_idx, block_size: int, scale: float = None, rows=None,
                          q_pos0: int = 0):
    """Reference outputs when each index entry names a micro-block of
    `block_size` consecutive tokens: the token operator applied to the
    expanded lists (block_idx [T, Hkv, n_blocks] -> [T, Hkv, n_blocks *
    block_size] token positions). Arguments otherwise as sparse_prefill."""
    block_idx = np.asarray(block_idx)
    R, Hkv, nb = block_idx.shape
    tokens = np.empty((R, Hkv, nb * block_size), dtype=np.int64)
    for i in range(R):
        for g in range(Hkv):
            tokens[i, g] = expand_blocks(block_idx[i, g], block_size)
    return sparse_prefill(q, k, v, tokens, scale=scale, rows=rows, q_pos0=q_pos0,
                          Hkv=np.asarray(k).shape[1])


def pool_selected_slots(slot_row, q_pos: int, slot_pos) -> list:
    """Slots a query at position q_pos (in its own request) attends to: the
    entries s of its list that name a pool slot (0 <= s < n_slots) holding a
    token (slot_pos[s] >= 0) at a position <= q_pos; list order, repeats kept."""
    n_slots = len(slot_pos)
    out = []
    for s in slot_row:
        s = int(s)
        if 0 <= s < n_slots and 0 <= int(slot_pos[s]) <= q_pos:
            out.append(s)
    return out


def sparse_prefill_pool(q, k_pool, v_pool, slot_idx, q_pos, slot_pos, scale: float = None, rows=None):
    """Reference outputs of a ragged batch over a K/V slot pool.

    q        [total_q, Hq, 256]  query rows of all requests, concatenated
    k_pool, v_pool [n_slots, Hkv, 256]
    slot_idx [total_q, Hkv, K]   pool slots (or [len(rows), Hkv, K] with rows)
    q_pos    [total_q]           position of each query row in its request
    slot_pos [n_slots]           position of the token held by each slot
    rows     optional query rows to evaluate

    Returns out float64 [R, Hq, 256] and lse float64 [R, Hq].
    """
    q = np.asarray(q)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    Hq, Hkv = q.shape[1], k_pool.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    slot_idx = np.asarray(slot_idx)
    q_pos = np.asarray(q_pos)
    slot_pos = np.asarray(slot_pos)
    if rows is None:
        rows = np.arange(q.shape[0])
        idx_rows = slot_idx
    else:
        rows = np.asarray(rows, dtype=np.int64)
        idx_rows = slot_idx if slot_idx.shape[0] == rows.size else slot_idx[rows]
    out = np.zeros((rows.size, Hq, D))
    lse = np.full((rows.size, Hq), -np.inf)
    for i, r in enumerate(rows):
        q_r = bf16_to_f64(q[r])
        for g in range(Hkv):
            sel = pool_selected_slots(idx_rows[i, g], int(q_pos[r]), slot_pos)
            k_sel = bf16_to_f64(k_pool[sel, g, :]) if sel else np.zeros((0, D))
            v_sel = bf16_to_f64(v_pool[sel, g, :]) if sel else np.zeros((0, D))
            for h in range(Hq):
                if kv_head_of(h, G) != g:
                    continue
                o, l, _ = attend(q_r[h], k_sel, v_sel, scale)
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
