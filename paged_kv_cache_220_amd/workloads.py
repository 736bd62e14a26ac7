"""Seeded synthetic decode batches for PagedAttention decode.

This module only draws random numbers, rounds them to the storage types and
builds block tables. It holds none of the attention arithmetic, so the HIP
path and the CPU oracle can both consume its output without sharing any of
the method's code.

Shapes follow the pages:
  * q            [num_seqs, num_heads, head_dim]                  (vLLM PagedAttention page, kernel pseudocode, argument list)
  * k/v cache    [num_blocks, num_kv_heads, head_dim, block_size] (same listing; the head axis is the KV-head axis,
                                                                   as the KV-cache size formula on the inference-optimisation page counts kv heads)
  * block_tables [num_seqs, max_blocks_per_seq] -> physical block id
  * seq_lens     [num_seqs]

Every array is returned as its raw storage bits (float32, uint16 for bf16,
uint8 for fp8, packed uint8 for int4: two tokens per byte, the even token in
the low nibble) so that both sides see exactly the same bytes. An int4 batch
also carries float32 scales per (physical block, KV head) for K and V.

Seeds: workload ``cN`` uses ``numpy.random.default_rng([220, N])`` for the
sequence lengths, the pool placement and q (drawn in that order); K and V are
drawn in chunks from ``default_rng([220, N, stream, chunk])`` with stream 1 for
K and 2 for V, so large pools can be produced chunk by chunk.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

BLOCK_SIZE_DEFAULT = 16

# Storage-type tags shared by the binding, the tests and the oracle inputs.
F32 = "f32"
BF16 = "bf16"
E5M2 = "e5m2"
E4M3 = "e4m3"
INT4 = "int4"

_NP_STORAGE = {F32: np.float32, BF16: np.uint16, E5M2: np.uint8, E4M3: np.uint8, INT4: np.uint8}
ELEM_BYTES = {F32: 4, BF16: 2, E5M2: 1, E4M3: 1, INT4: 0.5}

# Quiet-NaN bit patterns used to poison memory the kernel must never read.
NAN_BITS = {F32: np.uint32(0x7FC00000).view(np.float32), BF16: np.uint16(0x7FC0), E5M2: np.uint8(0x7F),
            E4M3: np.uint8(0x7F)}

_CHUNK = 1 << 22  # elements per K/V generation chunk


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    scale: np.float32
    k_scale: np.float32
    v_scale: np.float32
    seq_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray    # int32 [S, max_blocks]
    q: np.ndarray               # storage bits [S, H, D]
    k_cache: np.ndarray         # storage bits [NB, Hkv, D, bs]
    v_cache: np.ndarray         # storage bits [NB, Hkv, D, bs]
    seed: tuple = ()
    poisoned: bool = False
    k_block_scales: Optional[np.ndarray] = None   # float32 [NB, Hkv] (int4 caches)
    v_block_scales: Optional[np.ndarray] = None

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def describe(self) -> Dict:
        return dict(workload=self.name, num_seqs=self.num_seqs, num_heads=self.num_heads,
                    num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, block_size=self.block_size,
                    q_dtype=self.q_dtype, kv_dtype=self.kv_dtype, num_blocks=self.num_blocks,
                    total_tokens=int(self.seq_lens.sum()), max_seq_len=self.max_seq_len,
                    seed=list(self.seed))


# ----------------------------------------------------------------------------
# rounding to storage types (library conversions, round-to-nearest-even)
# ----------------------------------------------------------------------------

def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type and return raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    t = torch.from_numpy(x)
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == E5M2:
        return t.to(torch.float8_e5m2).view(torch.uint8).numpy()
    if dtype == E4M3:
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _normal_chunked(shape, seed_root, stream: int, dtype: str) -> np.ndarray:
    """N(0,1) draws of `shape`, rounded to `dtype`, chunk by chunk from child seeds.

    Chunk c always comes from default_rng(seed_root + [stream, c]), so the
    result does not depend on how many threads fill it.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=_NP_STORAGE[dtype])

    def fill(c):
        start = c * _CHUNK
        stop = min(n, start + _CHUNK)
        rng = np.random.default_rng(list(seed_root) + [stream, c])
        out[start:stop] = to_storage(rng.standard_normal(stop - start, dtype=np.float32), dtype)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    workers = max(1, min(8, len(os.sched_getaffinity(0)), nchunks))
    if workers == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _pack_int4(codes: np.ndarray) -> np.ndarray:
    """Signed codes -8..7 [..., 2n] -> bytes [..., n], the even token in the low nibble."""
    u = (codes.astype(np.int16) & 0x0F).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def _int4_chunked(shape, seed_root, stream: int) -> np.ndarray:
    """int4 codes for a pool of `shape` [NB, Hkv, D, bs] (packed on the last axis).

    Each code is an N(0,1) draw times 7/3, rounded to the nearest integer and
    held to -8..7 (about three standard deviations fill the code range), drawn
    chunk by chunk like the float pools. Synthetic storage only: the values a
    cache would hold are code * scale, with the scales drawn separately.
    """
    flat = _normal_chunked(shape, seed_root, stream, F32).reshape(shape)
    codes = np.clip(np.rint(flat * np.float32(7.0 / 3.0)), -8, 7).astype(np.int8)
    return _pack_int4(codes)


def _block_scales(nb: int, hkv: int, seed_root, stream: int) -> np.ndarray:
    """float32 scales per (block, KV head), log-uniform in [1/8, 1/2]: blocks
    differ, so a scale applied to the wrong block shows in the output."""
    rng = np.random.default_rng(list(seed_root) + [stream, 1 << 20])
    return np.exp2(rng.uniform(-3.0, -1.0, size=(nb, hkv))).astype(np.float32)


def _blocks_needed(seq_lens: np.ndarray, bs: int) -> np.ndarray:
    return (seq_lens.astype(np.int64) + bs - 1) // bs


# ----------------------------------------------------------------------------
# pool placement strategies
# ----------------------------------------------------------------------------

def _scatter_tables(rng, seq_lens, bs, pool_blocks, max_blocks):
    """Each sequence's blocks drawn without replacement from a pool of `pool_blocks`."""
    need = _blocks_needed(seq_lens, bs)
    total = int(need.sum())
    assert pool_blocks >= total
    perm = rng.permutation(pool_blocks)[:total].astype(np.int32)
    tables = np.zeros((len(seq_lens), max_blocks), dtype=np.int32)
    off = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[off:off + n]
        off += n
    return tables


def _shared_prefix_tables(rng, seq_lens, bs, prefix_blocks, max_blocks):
    """First `prefix_blocks` logical blocks of every sequence map to one shared set."""
    need = _blocks_needed(seq_lens, bs)
    private = int(np.maximum(need - prefix_blocks, 0).sum())
    pool = prefix_blocks + private
    perm = rng.permutation(pool).astype(np.int32)
    shared = perm[:prefix_blocks]
    tables = np.zeros((len(seq_lens), max_blocks), dtype=np.int32)
    off = prefix_blocks
    for s, n in enumerate(need):
        k = min(int(n), prefix_blocks)
        tables[s, :k] = shared[:k]
        rest = int(n) - k
        tables[s, k:k + rest] = perm[off:off + rest]
        off += rest
    return tables, pool


# ----------------------------------------------------------------------------
# the five decode batches
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")

CONFIG_TITLES = {
    "c1": "tiny fp32 MHA decode: 4 seqs, 4/4 heads, D=64, bs=16, seq_lens {1,17,33,100}",
    "c2": "chat bf16 GQA decode: 128 seqs, 64/8 heads, D=128, bs=16, seq_lens U[256,512]",
    "c3": "long-context bf16 GQA decode: 16 seqs x 32768 tokens, 64/8 heads, D=128, bs=16",
    "c4": "skewed bf16 GQA decode: 256 seqs, 90% log-U[64,1024], 10% U[8192,32768], 64/8 heads, D=128",
    "c5": "fp8-e5m2 KV decode with shared 64-block prefix: 128 seqs x 4096 tokens, 64/8 heads, D=128",
}


def _seq_lens_for(name: str, rng, num_seqs: Optional[int], seq_len: Optional[int]) -> np.ndarray:
    if name == "c1":
        return np.array([1, 17, 33, 100], dtype=np.int32)
    if name == "c2":
        S = num_seqs or 128
        return rng.integers(256, 512, size=S, endpoint=True).astype(np.int32)
    if name == "c3":
        S = num_seqs or 16
        return np.full(S, seq_len or 32768, dtype=np.int32)
    if name == "c4":
        S = num_seqs or 256
        n_long = int(round(0.1 * S))
        n_short = S - n_long
        lo_hi = (8192, 32768) if seq_len is None else (max(1, seq_len // 4), seq_len)
        short = np.floor(np.exp(rng.uniform(math.log(64), math.log(1024), size=n_short))).astype(np.int32)
        long = rng.integers(lo_hi[0], lo_hi[1], size=n_long, endpoint=True).astype(np.int32)
        lens = np.concatenate([short, long])
        return lens[rng.permutation(S)].astype(np.int32)
    if name == "c5":
        S = num_seqs or 128
        return np.full(S, seq_len or 4096, dtype=np.int32)
    raise ValueError(name)


def batch_heads(name: str, kv_dtype: Optional[str] = None):
    """(num_heads, num_kv_heads, head_dim, q dtype, KV dtype) of batch `name`."""
    if name == "c1":
        H, Hkv, D, qd, kvd = 4, 4, 64, F32, F32
    elif name == "c5":
        H, Hkv, D, qd, kvd = 64, 8, 128, BF16, E5M2
    else:
        H, Hkv, D, qd, kvd = 64, 8, 128, BF16, BF16
    if kv_dtype:
        if qd != BF16 or kv_dtype not in (BF16, E5M2, E4M3, INT4):
            raise ValueError(f"{name} cannot take a {kv_dtype} cache")
        kvd = kv_dtype
    return H, Hkv, D, qd, kvd


def batch_seq_lens(name: str) -> np.ndarray:
    """The sequence lengths of full-size batch `name`, without drawing its tensors."""
    if name not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {name}")
    rng = np.random.default_rng([220, CONFIG_NAMES.index(name) + 1])
    return _seq_lens_for(name, rng, None, None)


def make_workload(name: str, *, num_seqs: Optional[int] = None, seq_len: Optional[int] = None,
                  poison: bool = False, seed_extra: int = 0, kv_dtype: Optional[str] = None) -> Workload:
    """Build decode batch `name` (c1..c5).

    `num_seqs` / `seq_len` shrink a configuration while keeping its head
    shapes, dtypes and placement rule (used for small parity cases).
    `kv_dtype` overrides the cache type of the bf16-q batches (c2..c5), e.g.
    "e4m3" for the fp8 batch in the other OCP format.
    `poison=True` fills every byte the kernel must not read (unreferenced pool
    blocks, tail slots past seq_len in the last block, and table padding,
    which then points at a dedicated NaN block) with NaN.
    """
    if name not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {name}")
    idx = CONFIG_NAMES.index(name) + 1
    seed_root = (220, idx) if seed_extra == 0 else (220, idx, 1000 + seed_extra)
    rng = np.random.default_rng(list(seed_root))
    bs = BLOCK_SIZE_DEFAULT
    H, Hkv, D, qd, kvd = batch_heads(name, kv_dtype)

    seq_lens = _seq_lens_for(name, rng, num_seqs, seq_len)
    S = len(seq_lens)
    need = _blocks_needed(seq_lens, bs)
    max_blocks = max(1, int(need.max()))
    total = int(need.sum())

    if name == "c1":
        tables = _scatter_tables(rng, seq_lens, bs, 64, max_blocks)
        pool = 64
    elif name == "c2":
        pool = int(math.ceil(1.25 * total))
        tables = _scatter_tables(rng, seq_lens, bs, pool, max_blocks)
    elif name == "c3":
        pool = total
        tables = _scatter_tables(rng, seq_lens, bs, pool, max_blocks)
    elif name == "c4":
        pool = int(math.ceil(1.1 * total))
        tables = _scatter_tables(rng, seq_lens, bs, pool, max_blocks)
    else:
        prefix = min(64, int(need.min()))
        tables, pool = _shared_prefix_tables(rng, seq_lens, bs, prefix, max_blocks)

    if poison:
        pool += 1  # one extra, never referenced block that table padding points at

    q_f = rng.standard_normal((S, H, D), dtype=np.float32)
    q = to_storage(q_f, qd)
    ks = vs = None
    if kvd == INT4:
        k = _int4_chunked((pool, Hkv, D, bs), seed_root, 1)
        v = _int4_chunked((pool, Hkv, D, bs), seed_root, 2)
        ks = _block_scales(pool, Hkv, seed_root, 1)
        vs = _block_scales(pool, Hkv, seed_root, 2)
    else:
        k = _normal_chunked((pool, Hkv, D, bs), seed_root, 1, kvd)
        v = _normal_chunked((pool, Hkv, D, bs), seed_root, 2, kvd)

    if poison:
        _apply_poison(tables, seq_lens, need, k, v, kvd, bs, poison_block=pool - 1, k_scales=ks, v_scales=vs)

    one = np.float32(1.0)
    return Workload(name=name, num_seqs=S, num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                    q_dtype=qd, kv_dtype=kvd, scale=np.float32(1.0 / math.sqrt(D)), k_scale=one,
                    v_scale=one, seq_lens=seq_lens, block_tables=tables, q=q, k_cache=k, v_cache=v,
                    seed=seed_root, poisoned=poison, k_block_scales=ks, v_block_scales=vs)


def _apply_poison(tables, seq_lens, need, k, v, kvd, bs, poison_block, k_scales=None, v_scales=None):
    referenced = np.zeros(k.shape[0], dtype=bool)
    for s, n in enumerate(need):
        referenced[tables[s, :n]] = True
    unref = ~referenced
    if kvd == INT4:
        # int4 codes have no NaN: unread blocks get NaN scales and the most
        # negative code; tail slots get the most negative code (0x8 nibbles)
        k_scales[unref] = np.nan
        v_scales[unref] = np.nan
        k[unref] = 0x88
        v[unref] = 0x88
    else:
        nan = NAN_BITS[kvd]
        k[unref] = nan
        v[unref] = nan
    for s, (L, n) in enumerate(zip(seq_lens, need)):
        tables[s, n:] = poison_block
        if n > 0 and L % bs:
            last = tables[s, n - 1]
            if kvd == INT4:
                t0 = L % bs
                for t in range(t0, bs):
                    mask = np.uint8(0x0F if t % 2 == 0 else 0xF0)
                    k[last, :, :, t // 2] = (k[last, :, :, t // 2] & ~mask) | (np.uint8(0x88) & mask)
                    v[last, :, :, t // 2] = (v[last, :, :, t // 2] & ~mask) | (np.uint8(0x88) & mask)
            else:
                k[last, :, :, L % bs:] = nan
                v[last, :, :, L % bs:] = nan
    # A shared block may be the partial last block of one sequence and a full
    # block of another; poisoning its tail then changes valid data. The
    # placements here never do that (shared prefixes are whole blocks).


def workload_from_arrays(name, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads,
                         q_dtype, kv_dtype, scale=None, block_size=BLOCK_SIZE_DEFAULT,
                         k_block_scales=None, v_block_scales=None) -> Workload:
    """Wrap hand-built arrays (edge cases) in a Workload."""
    S, H, D = q.shape
    one = np.float32(1.0)
    sc = np.float32(1.0 / math.sqrt(D)) if scale is None else np.float32(scale)
    return Workload(name=name, num_seqs=S, num_heads=H, num_kv_heads=num_kv_heads, head_dim=D,
                    block_size=block_size, q_dtype=q_dtype, kv_dtype=kv_dtype, scale=sc, k_scale=one,
                    v_scale=one, seq_lens=np.asarray(seq_lens, dtype=np.int32),
                    block_tables=np.asarray(block_tables, dtype=np.int32), q=q, k_cache=k_cache,
                    v_cache=v_cache, k_block_scales=k_block_scales, v_block_scales=v_block_scales)


def random_edge_workload(seed: int, S: int, H: int, Hkv: int, D: int, seq_lens, q_dtype=BF16,
                         kv_dtype=BF16, extra_pool: int = 3, bs: int = BLOCK_SIZE_DEFAULT) -> Workload:
    """Small random batch with explicit lengths (zero-length and ragged cases)."""
    rng = np.random.default_rng([220, 99, seed])
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = _blocks_needed(seq_lens, bs)
    max_blocks = max(1, int(need.max()) if need.size else 1)
    pool = int(need.sum()) + extra_pool
    tables = _scatter_tables(rng, seq_lens, bs, pool, max_blocks)
    q = to_storage(rng.standard_normal((S, H, D), dtype=np.float32), q_dtype)
    if kv_dtype == INT4:
        seed_root = (220, 99, seed)
        k = _int4_chunked((pool, Hkv, D, bs), seed_root, 1)
        v = _int4_chunked((pool, Hkv, D, bs), seed_root, 2)
        return workload_from_arrays(f"edge{seed}", q, k, v, tables, seq_lens, Hkv, q_dtype, kv_dtype,
                                    k_block_scales=_block_scales(pool, Hkv, seed_root, 1),
                                    v_block_scales=_block_scales(pool, Hkv, seed_root, 2))
    k = to_storage(rng.standard_normal((pool, Hkv, D, bs), dtype=np.float32), kv_dtype)
    v = to_storage(rng.standard_normal((pool, Hkv, D, bs), dtype=np.float32), kv_dtype)
    return workload_from_arrays(f"edge{seed}", q, k, v, tables, seq_lens, Hkv, q_dtype, kv_dtype)


def permute_pool(w: Workload, seed: int) -> Workload:
    """Relabel physical blocks by a random permutation and rewrite the tables to match."""
    rng = np.random.default_rng([220, 77, seed])
    nb = w.num_blocks
    pi = rng.permutation(nb).astype(np.int32)       # old id -> new id
    k = np.empty_like(w.k_cache)
    v = np.empty_like(w.v_cache)
    k[pi] = w.k_cache
    v[pi] = w.v_cache
    ks = vs = None
    if w.k_block_scales is not None:
        ks = np.empty_like(w.k_block_scales)
        vs = np.empty_like(w.v_block_scales)
        ks[pi] = w.k_block_scales
        vs[pi] = w.v_block_scales
    return dataclasses.replace(w, name=w.name + "-perm", k_cache=k, v_cache=v, k_block_scales=ks,
                               v_block_scales=vs, block_tables=pi[w.block_tables].astype(np.int32))
