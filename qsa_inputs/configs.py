"""The five synthetic workloads of the QSA sparse-prefill operator.

Each workload is one prefill sequence of T tokens (query row t sits at
absolute position t, no cached prefix), head dim 256, bf16 Q/K/V drawn from
N(0, 1), scale 1/16 (= 1/sqrt(256), the "original D256 scale" kept by the
Ascend adapter in "Qwen4-Exp QSA llega al Ascend de Huawei", section "Lo que
realmente añade la pull request").

Index structure per (t, kv head), for rows with t + 1 > K:
  window  the last `window` positions ending at t,
  sink    position 0 (when `sink`),
  rest    K - window - sink distinct positions from the population
          [lo, t - window - gap], drawn uniformly or with weight
          1 / (1 + (t - s) / 1024),
then sorted ascending. Rows with t + 1 <= K select all of 0..t ascending and
pad with -1.

`gap` is 1 only for the tiny workload, whose random part is drawn from
[0, t - 32) while the window is the last 32 positions <= t, so position
t - 32 is never picked (taken literally).
"""
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

D = 256


@dataclass(frozen=True)
class Config:
    name: str
    number: int  # 1-based workload number, also the root seed
    T: int
    Hq: int
    Hkv: int
    K: int
    window: int
    sink: bool
    gap: int  # positions between the random population and the window
    sampler: str  # "uniform" or "weighted"
    outlier_frac: float = 0.0  # fraction of positions whose K and V rows are scaled
    outlier_scale: float = 1.0
    scale: float = 1.0 / 16.0
    oracle_rows: int = 0  # 0 = all rows; otherwise sampled rows for parity checks
    q_pos0: int = 0  # absolute position of query row 0 (tokens already cached)
    T_kv: int = 0  # K/V rows; 0 means T (no cached prefix)
    block_size: int = 1  # tokens named by one index entry (K, window, gap count entries)
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def kv_len(self) -> int:
        return self.T_kv if self.T_kv else self.T

    @property
    def n_rest(self) -> int:
        return self.K - self.window - (1 if self.sink else 0)

    def shapes(self) -> dict:
        return {
            "q": (self.T, self.Hq, D),
            "k": (self.kv_len, self.Hkv, D),
            "v": (self.kv_len, self.Hkv, D),
            "idx": (self.T, self.Hkv, self.K),
            "out": (self.T, self.Hq, D),
            "lse": (self.T, self.Hq),
        }

    @property
    def K_tokens(self) -> int:
        """Token slots per list: K entries of block_size tokens each."""
        return self.K * self.block_size

    def valid_slots(self) -> int:
        """Number of (t, kv head, token) slots that are valid (0 <= s <= position)."""
        if self.block_size > 1:
            return self._valid_block_slots()
        n = 0
        p0, p1, K = self.q_pos0, self.q_pos0 + self.T, self.K  # positions p0 .. p1-1
        ramp_end = min(p1, K)  # positions p < K select p + 1 slots
        if ramp_end > p0:
            n += (ramp_end * (ramp_end + 1) - p0 * (p0 + 1)) // 2
        n += max(0, p1 - max(p0, K)) * K
        return n * self.Hkv

    def _valid_block_slots(self) -> int:
        # Row t at position p sits in block b = p // B. Rows with b + 1 <= K
        # list every block 0..b: p + 1 valid tokens. Other rows list K blocks,
        # one of them b itself (the window ends at b): (K - 1) * B full blocks
        # plus the p % B + 1 tokens of b up to p.
        assert self.window >= 1, "block lists must hold the query's own block"
        B, K = self.block_size, self.K
        p = self.q_pos0 + np.arange(self.T, dtype=np.int64)
        dense = p // B + 1 <= K
        per_row = np.where(dense, p + 1, (K - 1) * B + p % B + 1)
        return int(per_row.sum()) * self.Hkv

    def gathered_bytes(self) -> int:
        """Algorithmic K+V bytes gathered: 512 B of K and 512 B of V per valid slot."""
        return self.valid_slots() * 2 * D * 2

    def useful_flops(self) -> int:
        """2*D flops for q.k plus 2*D for p*v, per valid slot and per query head."""
        return self.valid_slots() * self.G * 4 * D


CONFIGS: Tuple[Config, ...] = (
    Config(
        name="tiny_t256_h3x1_k64",
        number=1,
        T=256, Hq=3, Hkv=1, K=64,
        window=32, sink=False, gap=1, sampler="uniform",
        description="T=256, (Hq,Hkv)=(3,1), K=64: last 32 positions <= t plus 32 "
                    "distinct uniform positions from [0, t-32)",
    ),
    Config(
        name="t4096_h6x1_k512",
        number=2,
        T=4096, Hq=6, Hkv=1, K=512,
        window=128, sink=True, gap=0, sampler="uniform",
        description="T=4096, (6,1), K=512: 128-token window, sink 0, uniform rest",
    ),
    Config(
        name="t32768_h16x2_k2048_outliers",
        number=3,
        T=32768, Hq=16, Hkv=2, K=2048,
        window=256, sink=True, gap=0, sampler="weighted",
        outlier_frac=0.01, outlier_scale=8.0, oracle_rows=0,
        description="T=32768, (16,2), K=2048: 256-token window, sink 0, rest with "
                    "weight 1/(1+(t-s)/1024), independent per KV head; 1% of "
                    "positions have K and V rows scaled x8",
    ),
    Config(
        name="t32768_h24x2_k2048",
        number=4,
        T=32768, Hq=24, Hkv=2, K=2048,
        window=256, sink=True, gap=0, sampler="weighted",
        oracle_rows=0,
        description="T=32768, (24,2), K=2048: as the (16,2) workload without "
                    "outliers; 12 query heads per KV head",
    ),
    Config(
        name="long_t235008_h12x1_k2048",
        number=5,
        T=235008, Hq=12, Hkv=1, K=2048,
        window=512, sink=True, gap=0, sampler="uniform",
        oracle_rows=4096,
        description="T=235008 (the ~235K-token prefill rounded up to 918*256), "
                    "(12,1), K=2048: 512-token window, sink 0, uniform rest",
    ),
)

# The long-prefill operator case the pages test: 7,810 query tokens against a
# 65,536-token cache with 2,051 selected slots per query ("Nueve pruebas que
# pasaron" section). Read as the last 7,810 tokens of a 65,536-token sequence.
EXTEND_CONFIG = Config(
    name="extend_t7810_kv65536_h12x1_k2051",
    number=6,
    T=7810, Hq=12, Hkv=1, K=2051,
    window=512, sink=True, gap=0, sampler="uniform",
    oracle_rows=0, q_pos0=65536 - 7810, T_kv=65536,
    description="7,810 queries at positions 57,726..65,535 against a 65,536-token "
                "K/V cache, (12,1), K=2051: 512-token window, sink 0, uniform rest",
)

# Micro-block selection ("Por qué QSA es la parte incómoda, en cifras": the
# model's indexer has a compression ratio of 4 and selects 2,048 micro-blocks
# per query). K, window and gap count blocks; the weight law of the weighted
# sampler is 1 / (1 + (b_t - b) / 1024) in block units.
BLOCK_CONFIGS: Tuple[Config, ...] = (
    Config(
        name="blocks4_t256_h3x1_nb16",
        number=7,
        T=256, Hq=3, Hkv=1, K=16,
        window=4, sink=True, gap=0, sampler="uniform", block_size=4,
        description="T=256, (3,1), 16 micro-blocks of 4 tokens: the last 4 blocks "
                    "up to the query's own block, block 0, 11 uniform blocks",
    ),
    Config(
        name="blocks4_t32768_h24x2_nb2048",
        number=8,
        T=32768, Hq=24, Hkv=2, K=2048,
        window=64, sink=True, gap=0, sampler="weighted", block_size=4,
        oracle_rows=4096,
        description="T=32768, (24,2), 2,048 micro-blocks of 4 tokens (8,192 token "
                    "slots): 64-block window ending at the query's block, block 0, "
                    "rest weighted 1/(1+(b_t-b)/1024), independent per KV head",
    ),
)


@dataclass(frozen=True)
class Request:
    """One request of a ragged batch: `new` query tokens at positions
    cached .. cached + new - 1. Its first `cached` tokens are already in the
    pool: its own (share_from = -1) or the first `cached` tokens of request
    `share_from` (a shared prefix: the same slots)."""
    new: int
    cached: int = 0
    share_from: int = -1


@dataclass(frozen=True)
class PoolConfig:
    """A ragged batch of requests over one K/V slot pool. Every token of every
    request owns one slot, except shared-prefix tokens, which use the slots of
    the request they are shared from; `free_slots` more slots hold no token.
    Slots are assigned by a seeded random permutation (physical slots in no
    order). Per-query index lists follow the token recipe of Config over the
    query's own request, then name the slots of the chosen positions."""
    name: str
    number: int
    requests: Tuple[Request, ...]
    Hq: int
    Hkv: int
    K: int
    window: int
    sink: bool
    sampler: str
    free_slots: int = 0
    gap: int = 0
    scale: float = 1.0 / 16.0
    oracle_rows: int = 0
    decode: bool = False  # one query per request, run through the decode call
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def total_q(self) -> int:
        return sum(r.new for r in self.requests)

    @property
    def T(self) -> int:  # query rows of the batch
        return self.total_q

    @property
    def n_tokens(self) -> int:
        """Distinct tokens held by the pool (shared prefixes counted once)."""
        return sum(r.new + (r.cached if r.share_from < 0 else 0) for r in self.requests)

    @property
    def n_slots(self) -> int:
        return self.n_tokens + self.free_slots

    def valid_slots(self) -> int:
        n = 0
        for r in self.requests:
            p = r.cached + np.arange(r.new, dtype=np.int64)
            n += int(np.minimum(p + 1, self.K).sum())
        return n * self.Hkv

    def gathered_bytes(self) -> int:
        return self.valid_slots() * 2 * D * 2

    def useful_flops(self) -> int:
        return self.valid_slots() * self.G * 4 * D


# "Nueve pruebas que pasaron": physical slots in no order, two requests
# mapping a shared prefix, cache reuse.
POOL_CONFIGS: Tuple[PoolConfig, ...] = (
    PoolConfig(
        name="pool_4req_q311_h6x2_k64",
        number=9,
        requests=(Request(new=200), Request(new=77, cached=96, share_from=0),
                  Request(new=33, cached=150), Request(new=1)),
        Hq=6, Hkv=2, K=64, window=16, sink=True, sampler="uniform", free_slots=50,
        description="4 requests (200 new; 77 new after 96 tokens shared with the first; "
                    "33 new after 150 own cached; 1 new), (6,2), K=64, 50 empty slots",
    ),
    PoolConfig(
        name="pool_4req_q32768_h24x2_k2048",
        number=10,
        requests=(Request(new=12288), Request(new=8192, cached=8192, share_from=0),
                  Request(new=6144, cached=16384), Request(new=6144)),
        Hq=24, Hkv=2, K=2048, window=256, sink=True, sampler="weighted",
        free_slots=16384, oracle_rows=0,
        description="32,768 query tokens in 4 requests over a 65,536-slot pool: "
                    "12,288 new; 8,192 new after the first 8,192 tokens of the first "
                    "request (shared slots); 6,144 new after 16,384 own cached; "
                    "6,144 new; 16,384 empty slots. (24,2), K=2048, 256 window, sink, "
                    "weighted rest",
    ),
    PoolConfig(
        name="pool_4req_q32768_slots245760_h24x2_k2048",
        number=13,
        requests=tuple(Request(new=8192, cached=49152) for _ in range(4)),
        Hq=24, Hkv=2, K=2048, window=256, sink=True, sampler="weighted",
        free_slots=16384, oracle_rows=0,
        description="32,768 query tokens in 4 requests of 8,192 new tokens after 49,152 "
                    "own cached ones each, over a 245,760-slot pool (16,384 empty). "
                    "(24,2), K=2048, 256 window, sink, weighted rest",
    ),
)


def _decode_requests(lengths, share_every):
    """One new token per request after lengths[r] - 1 cached tokens; every
    `share_every`-th request after the first has its whole cached prefix in
    common with request 0 (the same slots)."""
    reqs = []
    for r, L in enumerate(lengths):
        shared = r > 0 and share_every and r % share_every == 1 and L <= lengths[0]
        reqs.append(Request(new=1, cached=L - 1, share_from=0 if shared else -1))
    return tuple(reqs)


# Decode: one query token per request (the serving phase the pages leave out
# of their prefill path), lists over each request's whole context.
DECODE_CONFIGS: Tuple[PoolConfig, ...] = (
    PoolConfig(
        name="decode_4req_h6x2_k512",
        number=11,
        requests=(Request(new=1, cached=2499), Request(new=1, cached=999, share_from=0),
                  Request(new=1, cached=76), Request(new=1, cached=299)),
        Hq=6, Hkv=2, K=512, window=64, sink=True, sampler="uniform", free_slots=100, decode=True,
        description="4 requests decoding one token each after 2,499 / 999 (shared with the "
                    "first) / 76 / 299 cached tokens, (6,2), K=512, 100 empty slots",
    ),
    PoolConfig(
        name="decode_16req_ctx16k_64k_h24x2_k2048",
        number=12,
        requests=_decode_requests(tuple(65536 - 3276 * r for r in range(16)), share_every=4),
        Hq=24, Hkv=2, K=2048, window=256, sink=True, sampler="weighted", free_slots=8192, decode=True,
        description="16 requests decoding one token each, contexts 65,536 down to 16,396 "
                    "tokens (every fourth one sharing its prefix with the first), (24,2), "
                    "K=2048, 256 window, sink, weighted rest, 8,192 empty slots",
    ),
)

ALL_CONFIGS = CONFIGS + (EXTEND_CONFIG,) + BLOCK_CONFIGS + POOL_CONFIGS + DECODE_CONFIGS
_BY_NAME = {c.name: c for c in ALL_CONFIGS}
_BY_NUMBER = {c.number: c for c in ALL_CONFIGS}
assert len(_BY_NUMBER) == len(ALL_CONFIGS)


def get_config(key):
    """Look a workload up by 1-based number, by name, or by 'c<number>'."""
    if isinstance(key, (Config, PoolConfig)):
        return key
    if isinstance(key, int):
        return _BY_NUMBER[key]
    if isinstance(key, str):
        if key in _BY_NAME:
            return _BY_NAME[key]
        if key.startswith("c") and key[1:].isdigit():
            return get_config(int(key[1:]))
    raise KeyError(f"unknown workload {key!r}")
