"""Pins for the oracle's cache-writing side: the E5M2 and bf16 encoders
against torch's conversions (a library routine) and against the format's own
fixed points, and the paged append / block copy against their definitions
read back through the (separately pinned) logical reassembly."""

import math

import numpy as np
import pytest
import torch

from oracle import pa_oracle as O
from paged_kv_cache_220_amd import workloads as W


def _torch_e5m2(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def _torch_bf16(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _e5m2_ties():
    """Every midpoint between adjacent finite E5M2 values, and its float32 neighbours."""
    vals = np.array(sorted({O.e5m2_value(c) for c in range(0x7C)}))       # non-negative finite values
    mids = (vals[:-1] + vals[1:]) / 2
    mids = np.concatenate([mids, [(57344.0 + 65536.0) / 2]])                 # the overflow midpoint
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)                      # exact in float32
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    out = np.concatenate([m32, up, dn, vals.astype(np.float32)])
    return np.concatenate([out, -out])


def test_e5m2_encoder_matches_torch_random_and_ties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-9, 6, 300000)).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-40, 3e38], np.float32)
    x = np.concatenate([x, _e5m2_ties(), specials])
    assert np.array_equal(O.e5m2_encode(x.astype(np.float64)), _torch_e5m2(x))


def test_e5m2_encoder_fixed_points():
    codes = np.array([c for c in range(256) if not math.isnan(O.e5m2_value(c))], dtype=np.uint8)
    vals = O.decode_bits(codes, "e5m2")
    assert np.array_equal(O.e5m2_encode(vals), codes)                  # every value encodes to itself
    assert O.e5m2_encode(np.array([61440.0]))[0] == 0x7C               # tie at the top rounds to inf (even)
    assert O.e5m2_encode(np.array([61439.99]))[0] == 0x7B
    assert O.e5m2_encode(np.array([2.0 ** -17]))[0] == 0x00            # tie to even: zero
    assert O.e5m2_encode(np.array([3 * 2.0 ** -17]))[0] == 0x02


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-40, 38, 300000)).astype(np.float32)
    bits = rng.integers(0, 1 << 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, bits, np.array([0.0, -0.0, np.inf, -np.inf, 3.39e38, -3.4e38, 1 + 2 ** -8], np.float32)])
    ours, tor = O.bf16_encode(x), _torch_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], tor[~nan])
    assert np.all(np.isnan(O.decode_bits(ours[nan], "bf16")))


def _append_case(kv_dtype, in_dtype, seed=0):
    rng = np.random.default_rng([7, seed])
    w = W.random_edge_workload(seed, S=3, H=8, Hkv=2, D=64, seq_lens=[5, 16, 40], q_dtype="bf16",
                               kv_dtype=kv_dtype)
    # one new token per sequence at position seq_len (the slot after the last), plus a padding entry
    token_seq = np.array([0, 1, 2, 1], np.int32)
    token_pos = np.array([5, 16, 40, -1], np.int32)
    tables = w.block_tables.copy()
    need = (w.seq_lens + 1 + 15) // 16
    if tables.shape[1] < need.max():
        tables = np.pad(tables, ((0, 0), (0, int(need.max()) - tables.shape[1])))
    free = [b for b in range(w.num_blocks) if b not in set(tables.ravel().tolist())]
    for s in range(3):
        for j in range(need[s]):
            if j * 16 >= w.seq_lens[s]:
                tables[s, j] = free.pop()
    new = rng.standard_normal((4, 2, 64)).astype(np.float32)
    new_bits = W.to_storage(new, in_dtype)
    return w, tables, token_seq, token_pos, new_bits, W.to_storage(-new, in_dtype)


@pytest.mark.parametrize("kv_dtype,in_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"),
                                               ("e5m2", "bf16"), ("e5m2", "f32")])
def test_append_writes_exactly_the_new_slots(kv_dtype, in_dtype):
    w, tables, tseq, tpos, kn, vn = _append_case(kv_dtype, in_dtype)
    k2, v2 = O.paged_append(kn, vn, w.k_cache, w.v_cache, tables, tseq, tpos, in_dtype, kv_dtype)
    changed = np.zeros(w.k_cache.shape, bool)
    for i in range(3):
        s, p = tseq[i], tpos[i]
        changed[tables[s, p // 16], :, :, p % 16] = True
        # reading the sequence back through the table gives the new token's encoded row
        Lnew = int(p) + 1
        for g in range(2):
            K = O.logical_kv(k2, tables, s, Lnew, g, kv_dtype)
            ref = O.decode_bits(O.encode_bits(O.decode_bits(kn[i, g], in_dtype).astype(np.float32), kv_dtype),
                                kv_dtype)
            assert np.array_equal(K[-1], ref)
            assert np.array_equal(K[:-1], O.logical_kv(w.k_cache, tables, s, Lnew - 1, g, kv_dtype))
    same = lambda a, b: np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert same(k2[~changed], w.k_cache[~changed]) and same(v2[~changed], w.v_cache[~changed])


def test_append_quantises_value_over_scale():
    w, tables, tseq, tpos, kn, vn = _append_case("e5m2", "f32")
    k2, _ = O.paged_append(kn, vn, w.k_cache, w.v_cache, tables, tseq, tpos, "f32", "e5m2", k_scale=0.37)
    s, p = tseq[0], tpos[0]
    got = k2[tables[s, p // 16], :, :, p % 16]
    want = _torch_e5m2(kn[0] / np.float32(0.37))
    assert np.array_equal(got, want)


def test_copy_blocks_definition():
    w = W.make_workload("c5", num_seqs=2, seq_len=1100)
    src = np.array([3, 7, 11], np.int32)
    dst = np.array([60, 5, 70], np.int32)
    k2, v2 = O.copy_blocks(w.k_cache, w.v_cache, src, dst)
    for a, b in zip(src, dst):
        assert np.array_equal(k2[b], w.k_cache[a]) and np.array_equal(v2[b], w.v_cache[a])
    keep = np.setdiff1d(np.arange(w.num_blocks), dst)
    assert np.array_equal(k2[keep], w.k_cache[keep]) and np.array_equal(v2[keep], w.v_cache[keep])


# ------------------------------------------------------------------ E4M3 ----

def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_table_two_ways():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_bits(codes, "e4m3")
    tor = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(tor))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], tor[fin])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9 and O.e4m3_value(0x38) == 1.0
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))


def test_e4m3_encoder_matches_torch_random_and_ties():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-5, 3.5, 300000)).astype(np.float32)
    vals = np.array(sorted({O.e4m3_value(c) for c in range(0x7F)}))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    edges = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                            vals.astype(np.float32), [464.0, 464.01, 479.0, 480.0, 1e6, 0.0, -0.0, np.inf, -np.inf,
                                                      np.nan, 2.0 ** -10, 3 * 2.0 ** -10]])
    x = np.concatenate([x, edges.astype(np.float32), -edges.astype(np.float32)])
    assert np.array_equal(O.e4m3_encode(x.astype(np.float64)), _torch_e4m3(x))
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.decode_bits(codes, "e4m3")), codes)
