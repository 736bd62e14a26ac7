"""Pins of the oracle on inputs far from unit scale (no GPU).

The fp8 and int4 caches feed 16-bit matrix operands, so the GPU tests take
q scaled by 2^17 (past the binary16 range) and 2^-20 (into its subnormals)
and per-block scales of 2^+-18 ("vLLM e PagedAttention", the fp8_e5m2 KV flag;
"Optimização da inferência", the exercise comparing FP16, FP8 and INT4 KV
caches). The oracle computes in float64, where all of these are ordinary
numbers; these tests pin what it returns there against facts fixed by the
mathematics, not by the oracle's formulas:
  * a power-of-two factor on every V scale scales the output by that factor,
    exactly; one on every K scale, undone in the score scale, changes nothing;
  * when the top score beats every other by more than float64's exp range,
    softmax is one-hot: the output is that token's V row, bit for bit;
  * mixed per-block scales against attention written out token by token.
"""

import math

import numpy as np
import pytest
import torch

from oracle import pa_oracle as O
from paged_kv_cache_220_amd import workloads as W


def _scaled_q(w, power):
    """q times 2^power (exact for bf16 inside its exponent range)."""
    qf = (w.q.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** power)
    assert np.all(np.isfinite(qf))
    return W.to_storage(qf, "bf16")


def _run(w, q=None, ks=None, vs=None, scale=None):
    return O.paged_decode(w.q if q is None else q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                          w.num_kv_heads, w.scale if scale is None else scale, w.q_dtype, w.kv_dtype,
                          k_block_scales=w.k_block_scales if ks is None else ks,
                          v_block_scales=w.v_block_scales if vs is None else vs)


def _values(bits, kv_dtype):
    """Cache bits -> float64 through torch's conversions (independent of the oracle's tables)."""
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if kv_dtype == "e5m2":
        return t.view(torch.float8_e5m2).to(torch.float64).numpy()
    if kv_dtype == "e4m3":
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["e5m2", "int4"])
@pytest.mark.parametrize("power", [18, -18])
def test_v_scale_power_of_two_scales_output_exactly(kv_dtype, power):
    w = W.make_workload("c5", num_seqs=3, seq_len=300, kv_dtype=kv_dtype)
    ks = np.ones((w.num_blocks, w.num_kv_heads), np.float32) if w.k_block_scales is None else w.k_block_scales
    vs = np.ones((w.num_blocks, w.num_kv_heads), np.float32) if w.v_block_scales is None else w.v_block_scales
    base = _run(w, ks=ks, vs=vs)
    big = _run(w, ks=ks, vs=(vs * np.float32(2.0 ** power)).astype(np.float32))
    assert np.array_equal(big, base * 2.0 ** power)


@pytest.mark.parametrize("power", [18, -18])
def test_k_scale_power_of_two_undone_by_the_score_scale(power):
    w = W.make_workload("c5", num_seqs=3, seq_len=300, kv_dtype="int4")
    base = _run(w)
    moved = _run(w, ks=(w.k_block_scales * np.float32(2.0 ** power)).astype(np.float32),
                 scale=np.float32(w.scale * np.float32(2.0 ** -power)))
    assert np.array_equal(moved, base)


def test_huge_q_gives_the_top_token_v_row():
    """q x 2^17: scores of order 10^5, so every weight but the top one is
    exp(-gap) with gap > 745 and underflows to 0 in float64."""
    w = W.make_workload("c5", num_seqs=3, seq_len=500, kv_dtype="e5m2")
    q = _scaled_q(w, 17)
    out = _run(w, q=q)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sc = float(np.float32(w.scale))
    G = w.num_heads // w.num_kv_heads
    checked = 0
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for h in range(w.num_heads):
            g = h // G
            scores, rows = [], []
            for t in range(L):                       # token by token through the table
                b, slot = int(w.block_tables[s, t // 16]), t % 16
                kt = _values(w.k_cache[b, g, :, slot], "e5m2")
                scores.append(sc * math.fsum(float(a) * float(c) for a, c in zip(qf[s, h], kt)))
                rows.append(_values(w.v_cache[b, g, :, slot], "e5m2"))
            order = np.argsort(scores)
            if scores[order[-1]] - scores[order[-2]] <= 800.0:
                continue
            assert np.array_equal(out[s, h], rows[order[-1]])
            checked += 1
    assert checked >= w.num_seqs * w.num_heads // 2


def test_tiny_q_gives_nearly_the_mean_of_v():
    """q x 2^-20: scores below 1e-5, weights within 1e-5 of uniform, so the
    output is within 1e-5 * max|V| of the plain mean of the V rows."""
    w = W.make_workload("c5", num_seqs=2, seq_len=400, kv_dtype="e4m3")
    out = _run(w, q=_scaled_q(w, -20))
    G = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for g in range(w.num_kv_heads):
            rows = np.stack([_values(w.v_cache[int(w.block_tables[s, t // 16]), g, :, t % 16], "e4m3")
                             for t in range(L)])
            mean = rows.mean(axis=0)
            for h in range(g * G, (g + 1) * G):
                assert np.max(np.abs(out[s, h] - mean)) <= 1e-5 * np.abs(rows).max()


def test_mixed_extreme_block_scales_token_by_token():
    """Per-block K and V scales 2^U(-18, 18) (not powers of two) on a tiny
    fp8 cache against attention written out with Python floats."""
    w = W.random_edge_workload(61, S=2, H=4, Hkv=2, D=128, seq_lens=[37, 70], kv_dtype="e5m2")
    rng = np.random.default_rng(62)
    ks = np.exp2(rng.uniform(-18, 18, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
    vs = np.exp2(rng.uniform(-18, 18, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
    out = _run(w, ks=ks, vs=vs)
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sc = float(np.float32(w.scale))
    G = w.num_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for h in range(w.num_heads):
            g = h // G
            scores, rows = [], []
            for t in range(L):
                b, slot = int(w.block_tables[s, t // 16]), t % 16
                kt = _values(w.k_cache[b, g, :, slot], "e5m2") * float(ks[b, g])
                scores.append(sc * math.fsum(float(a) * float(c) for a, c in zip(qf[s, h], kt)))
                rows.append(_values(w.v_cache[b, g, :, slot], "e5m2") * float(vs[b, g]))
            top = max(scores)
            wts = [math.exp(x - top) for x in scores]
            tot = math.fsum(wts)
            want = np.array([math.fsum(wt * r[d] for wt, r in zip(wts, rows)) / tot for d in range(128)])
            unit = max(float(np.abs(r).max()) for r in rows)
            assert np.max(np.abs(out[s, h] - want)) <= 1e-12 * unit
