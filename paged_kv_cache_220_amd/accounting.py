"""Byte and flop accounting for PagedAttention decode.

The per-token KV size follows the KV-cache memory formula on the
"Optimização da inferência" page ("Caches de KV"): 2 (K and V) x layers x KV
heads x head_dim x bytes per element. For one attention layer this is
2 * Hkv * D * elem_bytes per token. The ops:byte figure follows the roofline
section of the same page ("O framework de operações:byte").
"""

from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "e5m2": 1, "e4m3": 1, "int4": 0.5}
BLOCK_SCALE_BYTES = 4   # one float32 scale per (block, KV head) for K and one for V (int4)


def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int, seq_len: int, elem_bytes: int) -> int:
    """Whole-model KV-cache size for one sequence of `seq_len` tokens."""
    return 2 * num_layers * num_kv_heads * head_dim * seq_len * elem_bytes


def kv_bytes_per_token_layer(num_kv_heads: int, head_dim: int, kv_dtype: str) -> int:
    return int(2 * num_kv_heads * head_dim * ELEM_BYTES[kv_dtype])


def algorithmic_kv_bytes(seq_lens, num_kv_heads: int, head_dim: int, kv_dtype: str, block_size: int = 16) -> int:
    """Token-exact K+V bytes one decode call must read (logical tokens); an int4
    cache adds its K and V scale of every logical block it reads."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    total = int(lens.sum()) * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_dtype)
    if kv_dtype == "int4":
        total += int(((lens + block_size - 1) // block_size).sum()) * 2 * num_kv_heads * BLOCK_SCALE_BYTES
    return total


def unique_kv_bytes(seq_lens, block_tables, num_kv_heads: int, head_dim: int, block_size: int, kv_dtype: str) -> int:
    """K+V bytes of the distinct physical blocks referenced (shared prefixes counted once)."""
    ids = set()
    for s, L in enumerate(np.asarray(seq_lens)):
        n = (int(L) + block_size - 1) // block_size
        ids.update(np.asarray(block_tables[s, :n]).tolist())
    return len(ids) * block_size * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_dtype)


def io_bytes(num_seqs: int, num_heads: int, head_dim: int, q_dtype: str, seq_lens, block_size: int) -> int:
    """q in, out written, the table entries that are read, and seq_lens."""
    qb = num_seqs * num_heads * head_dim * ELEM_BYTES[q_dtype]
    nblk = int(((np.asarray(seq_lens, dtype=np.int64) + block_size - 1) // block_size).sum())
    return 2 * qb + 4 * nblk + 4 * num_seqs


def flops(seq_lens, num_heads: int, head_dim: int) -> int:
    """QK and PV multiply-adds per token and query head: 4 * D flops."""
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * num_heads * 4 * head_dim


def ops_per_byte(peak_flops: float, peak_bytes_per_s: float) -> float:
    """Roofline crossover: compute roof / memory roof."""
    return peak_flops / peak_bytes_per_s
