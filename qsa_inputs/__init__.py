"""Seeded synthetic inputs for the QSA sparse-prefill operator.

This module only draws data: bf16 Q/K/V tensors and int32 top-K index
lists with the shapes and structure of the workloads the operator is run on.
It holds none of the operator's arithmetic (no scores, no softmax, no
weighted sums), so both the CPU oracle and the GPU path can consume the same
arrays without sharing any of the method.

Shapes follow the operator description in "Qwen4-Exp QSA llega al Ascend de
Huawei" (orcarouter.ai, Spanish page), section "Lo que realmente añade la
pull request": rotated Q, KV cache K/V with head dim 256 in bf16, and a
token-granular selection per (query token, KV head). The local head shapes
(3,1), (6,1), (12,1), (16,2), (24,2) come from the same section; the 2,048
selection budget and the 24-query / 2-KV-head model from section "Por qué
QSA es la parte incómoda, en cifras"; the ~235K long-prefill length from
"Rò rỉ Qwen 4: SGLang chia nhỏ Prefill của Qwen4Exp" (orcarouter.ai,
Vietnamese page), section "Các delta đo được".

Everything is NumPy on the host: arrays are returned as
  q   uint16 [T, Hq, 256]   bf16 bit patterns
  k   uint16 [T, Hkv, 256]  bf16 bit patterns
  v   uint16 [T, Hkv, 256]  bf16 bit patterns
  idx int32  [T, Hkv, K]    token positions, -1 padded
(micro-block numbers for the block workloads). Ragged batches over a K/V slot
pool come from `batch.make_pool_inputs`.
"""
from .configs import (
    ALL_CONFIGS,
    BLOCK_CONFIGS,
    CONFIGS,
    DECODE_CONFIGS,
    EXTEND_CONFIG,
    POOL_CONFIGS,
    Config,
    PoolConfig,
    Request,
    get_config,
)
from .batch import make_pool_inputs, sample_pool_rows, slot_tables
from .generate import (
    make_inputs,
    make_qkv,
    make_indices,
    sample_rows,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
)

__all__ = [
    "ALL_CONFIGS",
    "BLOCK_CONFIGS",
    "CONFIGS",
    "DECODE_CONFIGS",
    "EXTEND_CONFIG",
    "POOL_CONFIGS",
    "Config",
    "PoolConfig",
    "Request",
    "make_pool_inputs",
    "sample_pool_rows",
    "slot_tables",
    "get_config",
    "make_inputs",
    "make_qkv",
    "make_indices",
    "sample_rows",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]
