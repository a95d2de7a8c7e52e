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

    def valid_slots(self) -> int:
        """Number of (t, kv head, slot) entries that are valid (0 <= s <= position)."""
        n = 0
        p0, p1, K = self.q_pos0, self.q_pos0 + self.T, self.K  # positions p0 .. p1-1
        ramp_end = min(p1, K)  # positions p < K select p + 1 slots
        if ramp_end > p0:
            n += (ramp_end * (ramp_end + 1) - p0 * (p0 + 1)) // 2
        n += max(0, p1 - max(p0, K)) * K
        return n * self.Hkv

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
        outlier_frac=0.01, outlier_scale=8.0, oracle_rows=4096,
        description="T=32768, (16,2), K=2048: 256-token window, sink 0, rest with "
                    "weight 1/(1+(t-s)/1024), independent per KV head; 1% of "
                    "positions have K and V rows scaled x8",
    ),
    Config(
        name="t32768_h24x2_k2048",
        number=4,
        T=32768, Hq=24, Hkv=2, K=2048,
        window=256, sink=True, gap=0, sampler="weighted",
        oracle_rows=4096,
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
    oracle_rows=512, q_pos0=65536 - 7810, T_kv=65536,
    description="7,810 queries at positions 57,726..65,535 against a 65,536-token "
                "K/V cache, (12,1), K=2051: 512-token window, sink 0, uniform rest",
)

_BY_NAME = {c.name: c for c in CONFIGS + (EXTEND_CONFIG,)}


def get_config(key) -> Config:
    """Look a workload up by 1-based number, by name, or by 'c<number>'."""
    if isinstance(key, Config):
        return key
    if isinstance(key, int):
        return EXTEND_CONFIG if key == EXTEND_CONFIG.number else CONFIGS[key - 1]
    if isinstance(key, str):
        if key in _BY_NAME:
            return _BY_NAME[key]
        if key.startswith("c") and key[1:].isdigit():
            return get_config(int(key[1:]))
    raise KeyError(f"unknown workload {key!r}")
