"""CPU oracle for PagedAttention decode (test infrastructure).

This module is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does. It shares no code with the HIP library and imports nothing from
the ``paged_kv_cache_220_amd`` package: it takes plain NumPy arrays holding
the exact storage bits the GPU receives.

What is computed (all in float64):

  For every sequence s and query head h, with L = seq_lens[s] and
  kv head g = h // (num_heads // num_kv_heads):
      token t (0 <= t < L) lives in physical block block_tables[s, t // bs]
      at slot t % bs;  K_t = K_cache[block, g, :, slot],  V_t likewise;
      out[s, h] = sum_t softmax_t(scale * q[s,h] . K_t) * V_t ,
  and out[s, h] = 0 when L == 0.

Sources on the pages:
  * "vLLM e PagedAttention: serving high-throughput", PagedAttention kernel
    pseudocode: the argument layouts (Q [seqs, heads, head_dim];
    K/V cache [blocks, heads, head_dim, block_size]; block_tables
    [seqs, max_blocks]; seq_lens), the loop over ceil(seq_len / block_size)
    logical blocks through the block table, the score q . K_block / sqrt(d),
    and the online-softmax update (running max m, running sum l, rescaled o)
    ending in output = o / l.
  * "Optimização da inferência", step 2 (attention with the KV cache): the
    dense max-subtracted softmax attention; with one query row no mask applies.
  * Same page, "PagedAttention": logical sequence positions map through a page
    table to fixed-size pages anywhere in memory; pages of a shared prefix are
    stored once and referenced by many requests.
  * Same page, "Caches de KV": the cache is sized by the number of KV heads
    (grouped-query attention: 64 query heads share 8 KV heads for Llama 3 70B).
  * "Continuous Batching e PagedAttention no vLLM", section 3: physical blocks
    need not be consecutive, and the last block may be partly unused.
  * The fp8-e5m2 KV option appears only as the flag name ``fp8_e5m2`` on the
    vLLM page; its decoding follows the OCP 8-bit floating point format
    (1 sign, 5 exponent bits with bias 15, 2 mantissa bits, IEEE-style
    subnormals, infinities and NaNs). The inference page's exercise compares
    KV caches in other precisions; the OCP E4M3 format (bias 7, 3 mantissa
    bits, no infinities, one NaN pattern per sign) is the other fp8 option.

Readings where the pages are silent (each is also listed with the design notes):
  * tail slots of the last block (t >= L) do not exist and take no part in
    the softmax or in P.V; the pseudocode's whole-block sums are read this way;
  * query head h uses KV head h // G (consecutive query heads share a KV head);
  * the scale is an argument (the pages fix 1/sqrt(head_dim)); the oracle uses
    the float32 value the GPU receives, widened to float64;
  * L == 0 gives a zero output row;
  * fp8 values are checked against the stored bytes decoded exactly, times the
    per-tensor scales k_scale / v_scale;
  * INT4 (the inference page's exercise names INT4 KV quantisation and its
    roughly fourfold capacity over FP16, nothing more): symmetric 4-bit
    two's-complement codes -8..7, two tokens per byte along the token axis
    (the even token in the low nibble), one float32 scale per (physical
    block, KV head) for K and one for V, so a value is
    code * k_scale * k_block_scales[block, kv head]. The same per-block scales
    may also multiply an fp8 cache.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "decode_bits", "e5m2_value", "logical_kv", "paged_decode", "paged_decode_rows",
    "online_decode", "merge_partials", "softmax_state", "combine_states", "dense_attention",
    "e5m2_encode", "bf16_encode", "encode_bits", "paged_append", "copy_blocks",
    "paged_attention_multi", "e4m3_value", "e4m3_encode",
    "int4_pack", "int4_unpack", "int4_encode", "block_values",
]


# ----------------------------------------------------------------------------
# storage decoding (exact)
# ----------------------------------------------------------------------------

def e5m2_value(code: int) -> float:
    """Exact value of one OCP E5M2 byte from its bit fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 2) & 0x1F
    man = code & 0x3
    if exp == 0x1F:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * (man / 4.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + man / 4.0) * 2.0 ** (exp - 15)


_E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)


def e4m3_value(code: int) -> float:
    """Exact value of one OCP E4M3 (E4M3FN) byte: 4 exponent bits with bias 7,
    3 mantissa bits, no infinities; S.1111.111 is NaN."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def int4_unpack(packed: np.ndarray) -> np.ndarray:
    """Bytes [..., n] -> signed codes [..., 2n] (int8): byte j holds token 2j in
    its low nibble and token 2j + 1 in its high nibble, two's complement."""
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int8)
    hi = (b >> 4).astype(np.int8)
    nib = np.stack([lo, hi], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def int4_pack(codes: np.ndarray) -> np.ndarray:
    """Signed codes [..., 2n] in -8..7 -> bytes [..., n] (inverse of int4_unpack)."""
    c = np.asarray(codes, dtype=np.int16)
    if c.min(initial=0) < -8 or c.max(initial=0) > 7 or c.shape[-1] % 2:
        raise ValueError("int4 codes must lie in -8..7, an even number per row")
    u = (c & 0x0F).astype(np.uint8).reshape(c.shape[:-1] + (c.shape[-1] // 2, 2))
    return (u[..., 0] | (u[..., 1] << 4)).astype(np.uint8)


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits -> float64 values, exactly. For int4 the last axis is
    packed (two tokens per byte) and comes back unpacked, as the codes."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        with np.errstate(invalid="ignore"):
            return b.view(np.float32).astype(np.float64)
    if dtype == "e5m2":
        return _E5M2_TABLE[np.asarray(bits, dtype=np.uint8)]
    if dtype == "e4m3":
        return _E4M3_TABLE[np.asarray(bits, dtype=np.uint8)]
    if dtype == "int4":
        return int4_unpack(bits).astype(np.float64)
    raise ValueError(dtype)


def _tokens_per_row(cache_bits: np.ndarray, dtype: str) -> int:
    return cache_bits.shape[3] * (2 if dtype == "int4" else 1)


def block_values(cache_bits: np.ndarray, b: int, g: int, dtype: str, elem_scale: float = 1.0,
                 block_scales: Optional[np.ndarray] = None) -> np.ndarray:
    """Values of physical block b, KV head g: float64 [D, block_size], the stored
    codes times the per-tensor scale and, if given, the block's own scale."""
    out = decode_bits(cache_bits[b, g], dtype)
    if elem_scale != 1.0:
        out = out * float(elem_scale)
    if block_scales is not None:
        out = out * float(np.float32(block_scales[b, g]))
    return out


# ----------------------------------------------------------------------------
# logical reassembly through the block table
# ----------------------------------------------------------------------------

def logical_kv(cache_bits: np.ndarray, block_tables: np.ndarray, s: int, L: int, kvh: int,
               dtype: str, elem_scale: float = 1.0, block_scales: Optional[np.ndarray] = None) -> np.ndarray:
    """K or V of sequence s, KV head kvh, in logical token order: float64 [L, D].

    Token t is read from physical block block_tables[s, t // bs], slot t % bs.
    Only the ceil(L / bs) table entries that hold tokens are read.
    """
    bs = _tokens_per_row(cache_bits, dtype)
    D = cache_bits.shape[2]
    if L == 0:
        return np.zeros((0, D), dtype=np.float64)
    nblk = (L + bs - 1) // bs
    ids = np.asarray(block_tables[s, :nblk], dtype=np.int64)
    tiles = decode_bits(cache_bits[ids, kvh], dtype)  # [nblk, D, bs]
    if block_scales is not None:
        tiles = tiles * np.asarray(block_scales, dtype=np.float32)[ids, kvh].astype(np.float64)[:, None, None]
    out = np.transpose(tiles, (0, 2, 1)).reshape(nblk * bs, D)[:L]
    if elem_scale != 1.0:
        out = out * float(elem_scale)
    return out


# ----------------------------------------------------------------------------
# plain definition: two-pass softmax attention over the reassembled sequence
# ----------------------------------------------------------------------------

def dense_attention(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query row against L keys/values: max-subtracted softmax, then weights @ V."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    sc = scale * (K @ qv)
    w = np.exp(sc - np.max(sc))
    return (w @ V) / np.sum(w)


def _check_shapes(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads):
    S, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if k_cache.shape != v_cache.shape or k_cache.shape[1] != num_kv_heads or k_cache.shape[2] != D:
        raise ValueError("cache shape mismatch")
    if block_tables.shape[0] != S or len(seq_lens) != S:
        raise ValueError("table / seq_lens shape mismatch")
    return S, H, D, H // num_kv_heads


def paged_decode_rows(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                      q_dtype: str, kv_dtype: str, rows: Iterable[Tuple[int, int]],
                      k_scale: float = 1.0, v_scale: float = 1.0, k_block_scales=None,
                      v_block_scales=None) -> np.ndarray:
    """out[s, h, :] for the listed (s, h) pairs only: float64 [len(rows), D]."""
    S, H, D, G = _check_shapes(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads)
    sc64 = float(np.float32(scale))
    rows = list(rows)
    out = np.zeros((len(rows), D), dtype=np.float64)
    cache = {}
    for i, (s, h) in enumerate(rows):
        g = h // G
        key = (s, g)
        if key not in cache:
            cache.clear()
            L = int(seq_lens[s])
            cache[key] = (logical_kv(k_cache, block_tables, s, L, g, kv_dtype, k_scale, k_block_scales),
                          logical_kv(v_cache, block_tables, s, L, g, kv_dtype, v_scale, v_block_scales))
        K, V = cache[key]
        out[i] = dense_attention(decode_bits(q[s, h], q_dtype), K, V, sc64)
    return out


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                 q_dtype: str, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs: Optional[Sequence[int]] = None, k_block_scales=None, v_block_scales=None) -> np.ndarray:
    """Full output float64 [S, H, D] (rows of sequences not in `seqs` stay zero).

    All query heads of one KV head are done together: scores [G, L] = q_g @ K^T.
    """
    S, H, D, G = _check_shapes(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads)
    sc64 = float(np.float32(scale))
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        if L == 0:
            continue
        for g in range(num_kv_heads):
            K = logical_kv(k_cache, block_tables, s, L, g, kv_dtype, k_scale, k_block_scales)
            V = logical_kv(v_cache, block_tables, s, L, g, kv_dtype, v_scale, v_block_scales)
            qg = decode_bits(q[s, g * G:(g + 1) * G], q_dtype)          # [G, D]
            sc = sc64 * (qg @ K.T)                                        # [G, L]
            w = np.exp(sc - sc.max(axis=1, keepdims=True))
            out[s, g * G:(g + 1) * G] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------
# second implementation: streaming softmax states folded chunk by chunk
# ----------------------------------------------------------------------------
# The decode kernel on "vLLM e PagedAttention" (its kernel pseudocode) keeps a
# running maximum, a running sum and a rescaled output while it walks the
# sequence's blocks. The same quantity is written here as a fold over softmax
# states. A state (m, l, o) summarises a stretch of tokens: m is its largest
# score, l the sum of exp(score - m) and o the same weights times the V rows.
# Two states of disjoint stretches combine by rescaling both to the larger m;
# the attention output of a stretch is o / l. Because combining is exact up to
# rounding, stretches of any length, in any grouping, give the two-pass result.

_EMPTY_STATE = (-math.inf, 0.0, None)


def softmax_state(scores: np.ndarray, V: np.ndarray):
    """State (m, l, o) of one stretch of tokens: scores [n], V rows [n, D]."""
    if scores.size == 0:
        return _EMPTY_STATE
    m = float(scores.max())
    w = np.exp(scores - m)
    return m, float(w.sum()), w @ V


def combine_states(a, b):
    """State of the union of two disjoint stretches (log-sum-exp rule)."""
    if a[0] == -math.inf:
        return b
    if b[0] == -math.inf:
        return a
    top = max(a[0], b[0])
    fa, fb = math.exp(a[0] - top), math.exp(b[0] - top)
    return top, fa * a[1] + fb * b[1], fa * a[2] + fb * b[2]


def merge_partials(parts: List[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Output o / l of the union of several partition states (the merge the
    partition-split decode applies); an all-empty list gives zeros."""
    acc = _EMPTY_STATE
    for st in parts:
        acc = combine_states(acc, st)
    if acc[0] == -math.inf:
        return np.zeros_like(parts[0][2]) if parts and parts[0][2] is not None else np.zeros(0)
    return acc[2] / acc[1]


def online_decode(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                  q_dtype: str, kv_dtype: str, partition_blocks: Optional[int] = None,
                  k_scale: float = 1.0, v_scale: float = 1.0, k_block_scales=None,
                  v_block_scales=None, chunk_tokens: int = 16) -> np.ndarray:
    """Streaming form: each (sequence, head) folds the states of consecutive
    chunks of `chunk_tokens` tokens; with `partition_blocks` the sequence is
    first cut into partitions of that many blocks, each folded on its own, and
    the partition states are merged at the end."""
    S, H, D, G = _check_shapes(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads)
    bs = _tokens_per_row(k_cache, kv_dtype)
    sc64 = float(np.float32(scale))
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L == 0:
            continue
        span = partition_blocks * bs if partition_blocks else L
        for g in range(num_kv_heads):
            K = logical_kv(k_cache, block_tables, s, L, g, kv_dtype, k_scale, k_block_scales)
            V = logical_kv(v_cache, block_tables, s, L, g, kv_dtype, v_scale, v_block_scales)
            for h in range(g * G, (g + 1) * G):
                qv = decode_bits(q[s, h], q_dtype)
                parts = []
                for p0 in range(0, L, span):
                    st = _EMPTY_STATE
                    for c0 in range(p0, min(L, p0 + span), chunk_tokens):
                        c1 = min(L, p0 + span, c0 + chunk_tokens)
                        st = combine_states(st, softmax_state(sc64 * (K[c0:c1] @ qv), V[c0:c1]))
                    parts.append(st)
                out[s, h] = merge_partials(parts)
    return out


# ----------------------------------------------------------------------------
#
# "Optimização da inferência", "Caches de KV": when token N is generated, only
# its key and value are computed and appended to the cached ones (the KVCache
# update of step 1 writes them at the next positions). In the paged layout of
# the vLLM page the position t of sequence s lives in block
# block_tables[s][t // bs], slot t % bs. The fp8 cache stores E5M2 bytes
# (the vLLM page's fp8_e5m2 flag) of value / scale.
#
# "PagedAttention" on the same page: pages of a shared prefix are stored once
# and copied only when a request diverges (copy on write). copy_blocks is that
# copy: whole physical blocks, every KV head, K and V.

def e5m2_encode(x) -> np.ndarray:
    """Values (exactly representable in float64) -> OCP E5M2 codes.

    Round to nearest, ties to even; magnitudes that round past the largest
    finite value (57344) become infinity; NaN keeps its sign and becomes the
    all-ones NaN code. Follows the format: 5 exponent bits with bias 15, 2
    mantissa bits, subnormal step 2^-16.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x).astype(np.uint16) << 7)
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.uint16)
    fin = np.isfinite(a)
    m, e = np.frexp(np.where(fin, a, 0.0))          # a = m * 2^e, m in [0.5, 1)
    E = e.astype(np.int64) - 1                      # a = (2m) * 2^E, 2m in [1, 2)
    normal = fin & (a >= 2.0 ** -14)
    # normal: q = RNE(a / 2^(E-2)) in [4, 8]; 8 carries into the exponent
    q = np.round(np.where(normal, a, 0.0) / np.exp2(np.where(normal, E - 2, 0).astype(np.float64)))
    carry = q >= 8
    E2 = np.where(carry, E + 1, E)
    q2 = np.where(carry, 4, q)
    biased = E2 + 15
    norm_code = (biased << 2) | (q2.astype(np.int64) - 4)
    overflow = normal & (biased >= 31)
    code = np.where(normal & ~overflow, norm_code, code)
    # subnormal (and zero): q = RNE(a / 2^-16) in [0, 4]; 4 is the smallest normal code
    sub = fin & (a < 2.0 ** -14)
    code = np.where(sub, np.round(np.where(sub, a, 0.0) * 2.0 ** 16).astype(np.int64), code)
    code = np.where(overflow | (np.isinf(a)), 0x7C, code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code.astype(np.uint16) | sign).astype(np.uint8)


def e4m3_encode(x) -> np.ndarray:
    """Values (exact in float64) -> OCP E4M3 codes, round to nearest, ties to even.

    The format has no infinity: a magnitude that rounds past 448 (the tie at
    464 rounds to 448, which is even), an infinity or a NaN becomes the NaN
    code with the input's sign. Subnormal step 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x).astype(np.uint16) << 7)
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    fin = np.isfinite(a)
    m, e = np.frexp(np.where(fin, a, 0.0))
    E = e.astype(np.int64) - 1
    normal = fin & (a >= 2.0 ** -6)
    q = np.round(np.where(normal, a, 0.0) / np.exp2(np.where(normal, E - 3, 0).astype(np.float64)))   # [8, 16]
    carry = q >= 16
    E2 = np.where(carry, E + 1, E)
    q2 = np.where(carry, 8, q).astype(np.int64)
    biased = E2 + 7
    norm_code = (biased << 3) | (q2 - 8)
    nan_code = normal & (norm_code >= 0x7F)            # rounds to 480 or beyond: no such value
    code = np.where(normal & ~nan_code, norm_code, code)
    sub = fin & (a < 2.0 ** -6)
    code = np.where(sub, np.round(np.where(sub, a, 0.0) * 2.0 ** 9).astype(np.int64), code)
    code = np.where(nan_code | ~fin, 0x7F, code)
    return (code.astype(np.uint16) | sign).astype(np.uint8)


def bf16_encode(x) -> np.ndarray:
    """float32 values -> bfloat16 bits, round to nearest even (8 significant bits).

    Overflow past the largest finite bfloat16 rounds to infinity; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    sign = np.signbit(x)
    fin = np.isfinite(a) & (a > 0)
    m, e = np.frexp(np.where(fin, a, 1.0))
    E = e.astype(np.int64) - 1
    # bfloat16 keeps 8 significant bits down to 2^-126 (then subnormal, step 2^-133)
    step_exp = np.maximum(E, -126) - 7
    r = np.round(np.where(fin, a, 0.0) / np.exp2(step_exp.astype(np.float64))) * np.exp2(step_exp.astype(np.float64))
    r = np.where(fin, r, a)
    r = np.where(r > 3.3895313892515355e38, np.inf, r)        # past the largest finite bfloat16
    r = np.where(sign, -r, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0) | (sign.astype(np.uint16) << 15), bits)
    return bits.astype(np.uint16)


def int4_encode(y) -> np.ndarray:
    """Values (already divided by their scale) -> int4 codes (int8, unpacked):
    the nearest integer, ties to even, held to -8..7; NaN gives 0."""
    y = np.asarray(y, dtype=np.float64)
    r = np.rint(np.where(np.isnan(y), 0.0, y))
    return np.clip(r, -8, 7).astype(np.int8)


def encode_bits(values_f32: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """float32 values -> cache storage bits. The fp8 and int4 codes are taken of
    value / scale, the division done in float32 (one correctly rounded
    division). int4 codes come back unpacked (int8, one per value)."""
    v = np.asarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return v.copy()
    if dtype == "bf16":
        return bf16_encode(v)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (v / np.float32(scale)).astype(np.float64)
    if dtype == "e5m2":
        return e5m2_encode(y)
    if dtype == "e4m3":
        return e4m3_encode(y)
    if dtype == "int4":
        return int4_encode(y)
    raise ValueError(dtype)


def _write_token(cache, blk, slot, codes, dtype):
    """Store one token's codes [Hkv, D] at (blk, slot); int4 replaces one nibble."""
    if dtype != "int4":
        cache[blk, :, :, slot] = codes
        return
    byte = cache[blk, :, :, slot // 2]
    nib = (np.asarray(codes, dtype=np.int16) & 0x0F).astype(np.uint8)
    if slot % 2 == 0:
        cache[blk, :, :, slot // 2] = (byte & 0xF0) | nib
    else:
        cache[blk, :, :, slot // 2] = (byte & 0x0F) | (nib << 4)


def paged_append(k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos,
                 in_dtype: str, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                 k_block_scales=None, v_block_scales=None):
    """Write new tokens into copies of the caches; returns (k_cache', v_cache').

    Token i (K/V rows [num_kv_heads, head_dim] in k_new[i], v_new[i]) belongs to
    sequence token_seq[i] at logical position token_pos[i] >= 0; a negative
    position marks a padding entry that writes nothing. With per-block scales
    the code of KV head g is taken of value / (k_scale * k_block_scales[blk, g]),
    the product rounded to float32 first.
    """
    k_out, v_out = k_cache.copy(), v_cache.copy()
    bs = _tokens_per_row(k_cache, kv_dtype)
    for i in range(len(token_seq)):
        pos = int(token_pos[i])
        if pos < 0:
            continue
        blk = int(block_tables[int(token_seq[i]), pos // bs])
        kv = decode_bits(k_new[i], in_dtype).astype(np.float32)    # [Hkv, D], exact
        vv = decode_bits(v_new[i], in_dtype).astype(np.float32)
        for cache_out, x, sc, bsc in ((k_out, kv, k_scale, k_block_scales), (v_out, vv, v_scale, v_block_scales)):
            if bsc is None:
                codes = encode_bits(x, kv_dtype, sc)
            else:
                per_head = np.float32(sc) * np.asarray(bsc, dtype=np.float32)[blk]          # [Hkv], float32
                codes = np.stack([encode_bits(x[g], kv_dtype, per_head[g]) for g in range(x.shape[0])])
            _write_token(cache_out, blk, pos % bs, codes, kv_dtype)
    return k_out, v_out


def copy_blocks(k_cache, v_cache, src, dst, k_block_scales=None, v_block_scales=None):
    """Copies of the caches with physical block dst[i] replaced by block src[i].
    With per-block scales, returns them copied alike as a third and fourth item."""
    k_out, v_out = k_cache.copy(), v_cache.copy()
    ks_out = None if k_block_scales is None else np.array(k_block_scales, copy=True)
    vs_out = None if v_block_scales is None else np.array(v_block_scales, copy=True)
    for a, b in zip(np.asarray(src), np.asarray(dst)):
        k_out[int(b)] = k_cache[int(a)]
        v_out[int(b)] = v_cache[int(a)]
        if ks_out is not None:
            ks_out[int(b)] = k_block_scales[int(a)]
            vs_out[int(b)] = v_block_scales[int(a)]
    if ks_out is None:
        return k_out, v_out
    return k_out, v_out, ks_out, vs_out


# ----------------------------------------------------------------------------
# several query positions per sequence (chunked prefill, speculative verify)
# ----------------------------------------------------------------------------
#
# "Optimização da inferência", step 2: with more than one query row the
# attention adds a causal mask, -1e9 on the scores of keys past each query's
# own position: the q_len queries are the last q_len positions of the
# sequence, and query i may attend keys j <= L - q_len + i. The large negative
# addend only removes those keys from the softmax; here they are left out.
# Speculative decoding verifies several candidate tokens in one pass, and
# chunked prefill feeds a prompt in pieces (same page; vLLM page flags), which
# is this computation over the paged cache.

def paged_attention_multi(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                          q_dtype: str, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                          k_block_scales=None, v_block_scales=None) -> np.ndarray:
    """q [S, q_len, H, D] -> float64 [S, q_len, H, D].

    seq_lens[s] counts every token in the cache, the q_len new ones included.
    Query i of sequence s attends tokens t < seq_lens[s] - q_len + 1 + i (zero row if none).
    """
    S, QL, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // num_kv_heads
    sc64 = float(np.float32(scale))
    out = np.zeros((S, QL, H, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L == 0:
            continue
        for g in range(num_kv_heads):
            K = logical_kv(k_cache, block_tables, s, L, g, kv_dtype, k_scale, k_block_scales)
            V = logical_kv(v_cache, block_tables, s, L, g, kv_dtype, v_scale, v_block_scales)
            for i in range(QL):
                n = L - QL + 1 + i
                if n <= 0:
                    continue
                qg = decode_bits(q[s, i, g * G:(g + 1) * G], q_dtype)       # [G, D]
                sc = sc64 * (qg @ K[:n].T)
                w = np.exp(sc - sc.max(axis=1, keepdims=True))
                out[s, i, g * G:(g + 1) * G] = (w @ V[:n]) / w.sum(axis=1, keepdims=True)
    return out
