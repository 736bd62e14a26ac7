"""GPU parity of paged attention with several query positions per sequence
(speculative-decode verification, chunked prefill) against the oracle."""

import numpy as np
import pytest
import torch

from gpu_helpers import abs_attention_multi, check, log, upload
from oracle import pa_oracle as O
from paged_kv_cache_220_amd import binding as B
from paged_kv_cache_220_amd import workloads as W

pytestmark = pytest.mark.gpu


def _dev(bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e5m2).cuda()


CASES = [
    ("c2", dict(num_seqs=10), 2),                  # 8 heads x 2 positions: one column group
    ("c2", dict(num_seqs=6), 4),                   # two column groups
    ("c5", dict(num_seqs=4, seq_len=2100), 8),     # four column groups, fp8 cache
    ("c3", dict(num_seqs=2, seq_len=5000), 3),
    ("c2", dict(num_seqs=6), 8),                   # bf16, four full column groups
    ("c3", dict(num_seqs=2, seq_len=3000), 5),     # bf16, 40 columns: the last group part-filled
]


@pytest.mark.parametrize("name,kw,ql", CASES, ids=[f"{c[0]}-q{c[2]}" for c in CASES])
@pytest.mark.parametrize("ptok", [0, 64, 512])
def test_multi_query_parity(name, kw, ql, ptok):
    w = W.make_workload(name, **kw)
    rng = np.random.default_rng([ql, ptok])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = O.paged_attention_multi(q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.num_kv_heads, w.scale,
                                  "bf16", w.kv_dtype)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    out = torch.empty_like(qd)
    log(f"case multi-query {name}{kw} q_len={ql} P={ptok}")
    B.pa_decode(qd, _dev(w.k_cache, w.kv_dtype), _dev(w.v_cache, w.kv_dtype), torch.from_numpy(w.block_tables).cuda(),
                torch.from_numpy(w.seq_lens).cuda(), w.num_kv_heads, float(w.scale), out, partition_tokens=ptok,
                max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    check(got, ref, w, f"multi-query {name} q_len={ql} P={ptok}", a=a)


@pytest.mark.parametrize("ql", [2, 4])
def test_multi_query_two_waves_per_item(ql):
    w = W.make_workload("c5", num_seqs=3, seq_len=2500)
    rng = np.random.default_rng([ql, 77])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = O.paged_attention_multi(q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.num_kv_heads, w.scale,
                                  "bf16", w.kv_dtype)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    for ptok in (0, 256):
        out = torch.empty_like(qd)
        log(f"case multi-query two waves q_len={ql} P={ptok}")
        B.pa_decode(qd, _dev(w.k_cache, w.kv_dtype), _dev(w.v_cache, w.kv_dtype),
                    torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda(), w.num_kv_heads,
                    float(w.scale), out, partition_tokens=ptok, max_seq_len=w.max_seq_len, kernel="mfma",
                    waves_per_item=2)
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"multi-query 2 waves q_len={ql} P={ptok}", a=a)


def test_query_window_longer_than_sequence():
    """Early queries of a sequence shorter than the window see no token: zero rows."""
    w = W.random_edge_workload(3, S=4, H=16, Hkv=2, D=128, seq_lens=[1, 3, 70, 0])
    ql = 4
    rng = np.random.default_rng(8)
    q = W.to_storage(rng.standard_normal((4, ql, 16, 128), dtype=np.float32), "bf16")
    ref = O.paged_attention_multi(q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, 2, w.scale, "bf16", "bf16")
    a = abs_attention_multi(q, w, num_kv_heads=2)
    for ptok in (0, 64):
        qd = _dev(q, "bf16")
        out = torch.full_like(qd, float("nan"))
        B.pa_decode(qd, _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16"), torch.from_numpy(w.block_tables).cuda(),
                    torch.from_numpy(w.seq_lens).cuda(), 2, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(got[0, :3] == 0) and np.all(got[1, :1] == 0) and np.all(got[3] == 0)
        check(got, ref, w, f"short window P={ptok}", a=a)


def _multi_ref(w, q):
    """Oracle per sequence (keeps the fp64 work proportional to the case)."""
    return np.concatenate([O.paged_attention_multi(q[s:s + 1], w.k_cache, w.v_cache, w.block_tables[s:s + 1],
                                                   w.seq_lens[s:s + 1], w.num_kv_heads, w.scale, w.q_dtype,
                                                   w.kv_dtype) for s in range(w.num_seqs)])


QBLOCKS = [
    ("c2", dict(num_seqs=4), 16),                       # 128 (position, head) pairs: two full blocks of 64
    ("c3", dict(num_seqs=2, seq_len=2000), 33),         # 264 pairs: five blocks, the last with 8
    ("c5", dict(num_seqs=2, seq_len=1500), 24),         # fp8 cache, three blocks
]


@pytest.mark.parametrize("name,kw,ql", QBLOCKS, ids=[f"{c[0]}-q{c[2]}" for c in QBLOCKS])
def test_query_blocks(name, kw, ql):
    """More (position, head) pairs than one work item holds: items cover blocks
    of 64, each reading the KV head's tiles; grid and list schedules, 1 and 2
    waves per item, single and split partitions."""
    w = W.make_workload(name, **kw)
    rng = np.random.default_rng([ql, 91])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = _multi_ref(w, q)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    kd, vd = _dev(w.k_cache, w.kv_dtype), _dev(w.v_cache, w.kv_dtype)
    td, ld = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda()
    for ptok, sched, nw in ((0, "auto", 0), (256, "grid", 1), (256, "queue", 2), (4096, "grid", 2)):
        out = torch.full_like(qd, float("nan"))
        log(f"case query blocks {name}{kw} q_len={ql} P={ptok} {sched} waves={nw}")
        B.pa_decode(qd, kd, vd, td, ld, w.num_kv_heads, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len, kernel="mfma", schedule=sched, waves_per_item=nw)
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"query blocks {name} q_len={ql} P={ptok} {sched}",
              a=a)


def test_query_blocks_one_kv_head():
    """64 query heads sharing one KV head (group 64): two positions make two blocks."""
    w = W.random_edge_workload(61, S=3, H=64, Hkv=1, D=128, seq_lens=[700, 65, 2])
    ql = 2
    rng = np.random.default_rng(62)
    q = W.to_storage(rng.standard_normal((3, ql, 64, 128), dtype=np.float32), "bf16")
    ref = _multi_ref(w, q)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    for ptok in (0, 128):
        out = torch.full_like(qd, float("nan"))
        B.pa_decode(qd, _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16"), torch.from_numpy(w.block_tables).cuda(),
                    torch.from_numpy(w.seq_lens).cuda(), 1, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len)
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"one KV head, group 64, P={ptok}", a=a)


def test_prefill_chunk():
    """A 256-token prefill chunk of one sequence (32 query blocks) over a 1000-token cache."""
    w = W.random_edge_workload(64, S=1, H=64, Hkv=8, D=128, seq_lens=[1000])
    ql = 256
    rng = np.random.default_rng(63)
    q = W.to_storage(rng.standard_normal((1, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = _multi_ref(w, q)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    out = torch.full_like(qd, float("nan"))
    log(f"case prefill chunk q_len={ql} L={int(w.seq_lens[0])}")
    B.pa_decode(qd, _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16"), torch.from_numpy(w.block_tables).cuda(),
                torch.from_numpy(w.seq_lens).cuda(), w.num_kv_heads, float(w.scale), out,
                max_seq_len=int(w.seq_lens[0]))
    torch.cuda.synchronize()
    check(out.float().cpu().numpy().astype(np.float64), ref, w, "prefill chunk", a=a)


@pytest.mark.parametrize("ql", [2, 4, 8, 12])
def test_multi_query_int4(ql):
    """int4 cache with per-block scales, 1, 2 and 4 column groups and two query blocks."""
    w = W.make_workload("c2", num_seqs=5, kv_dtype="int4")
    rng = np.random.default_rng([ql, 95])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = np.concatenate([O.paged_attention_multi(q[s:s + 1], w.k_cache, w.v_cache, w.block_tables[s:s + 1],
                                                  w.seq_lens[s:s + 1], w.num_kv_heads, w.scale, "bf16", "int4",
                                                  k_block_scales=w.k_block_scales, v_block_scales=w.v_block_scales)
                          for s in range(w.num_seqs)])
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    sc = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    kd = torch.from_numpy(np.ascontiguousarray(w.k_cache)).cuda()
    vd = torch.from_numpy(np.ascontiguousarray(w.v_cache)).cuda()
    for ptok in (0, 128):
        out = torch.full_like(qd, float("nan"))
        log(f"case multi-query int4 q_len={ql} P={ptok}")
        B.pa_decode(qd, kd, vd, torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda(),
                    w.num_kv_heads, float(w.scale), out, partition_tokens=ptok, max_seq_len=w.max_seq_len,
                    k_block_scales=sc(w.k_block_scales), v_block_scales=sc(w.v_block_scales))
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"multi-query int4 q_len={ql} P={ptok}", a=a)


SHARE = [
    # kv dtype, per-block scales, query positions: 8 heads x q_len pairs in blocks of 64
    ("bf16", False, 16),    # two blocks: by default one item of two waves
    ("bf16", False, 24),    # three blocks: four waves, one idle; or two items of two waves
    ("bf16", False, 13),    # 104 pairs: the last wave's 32 pairs are 8 real ones and 24 past the end
    ("e5m2", False, 16),
    ("e4m3", True, 20),
    ("int4", True, 24),
]


@pytest.mark.parametrize("kv,scaled,ql", SHARE, ids=[f"{c[0]}{'-scaled' if c[1] else ''}-q{c[2]}" for c in SHARE])
def test_tile_sharing(kv, scaled, ql):
    """Waves of one work item take one query block each and share every K/V
    tile through LDS: partitions of 1, 2 and 4 tiles (fewer tiles than LDS
    stages), lengths shorter than the query window, both schedules. The result
    of a query does not depend on how many waves share its tiles: 1, 2, 4 and
    8 waves per item give the same bits."""
    w = W.random_edge_workload(70 + ql, S=4, H=64, Hkv=8, D=128, seq_lens=[1000, 65, 1, 300], kv_dtype=kv)
    rng = np.random.default_rng([ql, 71])
    if scaled and kv != "int4":
        w.k_block_scales = np.exp2(rng.uniform(-2, 2, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
        w.v_block_scales = np.exp2(rng.uniform(-2, 2, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
        w.k_scale, w.v_scale = np.float32(0.75), np.float32(1.25)
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = np.concatenate([O.paged_attention_multi(q[s:s + 1], w.k_cache, w.v_cache, w.block_tables[s:s + 1],
                                                  w.seq_lens[s:s + 1], w.num_kv_heads, w.scale, "bf16", kv,
                                                  k_scale=float(w.k_scale), v_scale=float(w.v_scale),
                                                  k_block_scales=w.k_block_scales,
                                                  v_block_scales=w.v_block_scales)
                          for s in range(w.num_seqs)])
    a = abs_attention_multi(q, w)
    dev = upload(w)
    qd = _dev(q, "bf16")
    outs = {}
    for ptok, sched, nw in ((0, "auto", 0), (64, "grid", 2), (128, "grid", 4), (128, "grid", 2), (128, "grid", 1),
                            (128, "grid", 8), (256, "queue", 8), (64, "grid", 1)):
        out = torch.full_like(qd, float("nan"))
        log(f"case tile sharing {kv} scaled={scaled} q_len={ql} P={ptok} {sched} waves={nw}")
        B.pa_decode(qd, dev["k"], dev["v"], dev["tables"], dev["seq_lens"], w.num_kv_heads, float(w.scale), out,
                    partition_tokens=ptok, max_seq_len=w.max_seq_len, kernel="mfma", schedule=sched,
                    waves_per_item=nw, k_scale=float(w.k_scale), v_scale=float(w.v_scale),
                    k_block_scales=dev["k_block_scales"], v_block_scales=dev["v_block_scales"])
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        check(got, ref, w, f"tile sharing {kv} q_len={ql} P={ptok} {sched} waves={nw}", a=a)
        outs[(ptok, nw)] = out.view(torch.int16).cpu().numpy()
    for nw in (2, 4, 8):
        assert np.array_equal(outs[(128, nw)], outs[(128, 1)]), f"{nw} waves sharing tiles differ from one block per item"


@pytest.mark.parametrize("kv", ["bf16", "e5m2", "int4"])
def test_tile_sharing_poisoned(kv):
    """Tile sharing over a pool whose unread blocks, tail slots and table padding
    hold NaN (int4: NaN block scales and code -8): nothing outside the causal
    window and the sequence may reach the output."""
    w = W.make_workload("c2", num_seqs=6, poison=True, kv_dtype=kv)
    ql = 12                                          # 96 pairs: two query blocks
    rng = np.random.default_rng([ql, 73])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = np.concatenate([O.paged_attention_multi(q[s:s + 1], w.k_cache, w.v_cache, w.block_tables[s:s + 1],
                                                  w.seq_lens[s:s + 1], w.num_kv_heads, w.scale, "bf16", kv,
                                                  k_block_scales=w.k_block_scales,
                                                  v_block_scales=w.v_block_scales)
                          for s in range(w.num_seqs)])
    a = abs_attention_multi(q, w)
    dev = upload(w)
    qd = _dev(q, "bf16")
    for ptok, nw in ((0, 0), (64, 2), (128, 4)):
        out = torch.full_like(qd, float("nan"))
        log(f"case tile sharing poisoned {kv} P={ptok} waves={nw}")
        B.pa_decode(qd, dev["k"], dev["v"], dev["tables"], dev["seq_lens"], w.num_kv_heads, float(w.scale), out,
                    partition_tokens=ptok, max_seq_len=w.max_seq_len, kernel="mfma", waves_per_item=nw,
                    k_block_scales=dev["k_block_scales"], v_block_scales=dev["v_block_scales"])
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"tile sharing poisoned {kv} P={ptok} waves={nw}",
              a=a)


SHARE_SHAPES = [
    # (H, Hkv, q_len, seq_lens): pair counts that are not multiples of 32, MHA, one KV head
    (40, 8, 13, [700, 130, 13, 12]),     # G 5: 65 pairs -> 3 waves of 32, the last with 1 pair
    (8, 8, 100, [100, 257, 64]),         # MHA, 100 pairs, windows as long as the sequences
    (32, 1, 3, [900, 2, 0]),             # one KV head, 96 pairs; an empty sequence
]


@pytest.mark.parametrize("H,Hkv,ql,lens", SHARE_SHAPES, ids=[f"H{c[0]}-Hkv{c[1]}-q{c[2]}" for c in SHARE_SHAPES])
def test_tile_sharing_shapes(H, Hkv, ql, lens):
    w = W.random_edge_workload(80 + ql, S=len(lens), H=H, Hkv=Hkv, D=128, seq_lens=lens)
    rng = np.random.default_rng([ql, 81])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = _multi_ref(w, q)
    a = abs_attention_multi(q, w)
    qd = _dev(q, "bf16")
    kd, vd = _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16")
    td, ld = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda()
    for ptok, nw in ((0, 0), (64, 2), (128, 4), (256, 8), (128, 1)):
        out = torch.full_like(qd, float("nan"))
        log(f"case tile sharing shape H={H} Hkv={Hkv} q_len={ql} P={ptok} waves={nw}")
        B.pa_decode(qd, kd, vd, td, ld, w.num_kv_heads, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len, kernel="mfma", waves_per_item=nw)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        check(got, ref, w, f"tile sharing H={H} Hkv={Hkv} q_len={ql} P={ptok} waves={nw}", a=a)
        if 0 in lens:
            assert np.all(got[lens.index(0)] == 0)


HEAVY_LENS = [9000, 8200, 6000, 4101]


@pytest.mark.parametrize("ql", [4, 16])
def test_every_block_counted_once(ql):
    """Long sequences where one block holds V = 32 and q is tiny (weights all but
    uniform): the output then sits near 32 x 16 / n, and a kernel that skips the
    block, or takes it twice, misses by about that much, far beyond the gate.
    The heavy block is the first one, one in the middle of a partition, the
    first of the second 4096-token partition, and the last, partly filled one;
    4 positions run two column groups per wave, 16 share tiles between waves.
    (Elsewhere the gate with several positions, 2^-8 of the attention over |V|,
    is loose enough on sequences of several thousand tokens to let one
    ordinary block go unnoticed.)"""
    w = W.random_edge_workload(90 + ql, S=len(HEAVY_LENS), H=64, Hkv=8, D=128, seq_lens=HEAVY_LENS)
    heavy = [0, 100, 256, (HEAVY_LENS[3] - 1) // 16]
    for s, b in enumerate(heavy):
        w.v_cache[int(w.block_tables[s, b])] = W.to_storage(np.full(w.v_cache.shape[1:], 32.0, np.float32), "bf16")
    rng = np.random.default_rng([ql, 93])
    qf = rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32) * np.float32(2.0 ** -20)
    q = W.to_storage(qf, "bf16")
    ref = _multi_ref(w, q)
    a = abs_attention_multi(q, w)
    # tokens of each heavy block inside its sequence (the last one is partial)
    ntok = [min(16, HEAVY_LENS[s] - 16 * b) for s, b in enumerate(heavy)]
    assert ntok[3] == 5
    # the last query of each sequence attends all of it: missing the heavy block
    # there moves every element by about 32 x ntok / L, several times the gate
    gate = 2.0 ** -7 * np.abs(ref) + 2.0 ** -8 * a + 1e-4
    for s in range(w.num_seqs):
        assert gate[s, -1].max() < 0.25 * 32.0 * ntok[s] / HEAVY_LENS[s], f"sequence {s}: gate too loose"
    qd = _dev(q, "bf16")
    kd, vd = _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16")
    td, ld = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda()
    for ptok, nw in ((0, 0), (4096, 0), (512, 2)):
        out = torch.full_like(qd, float("nan"))
        log(f"case heavy block q_len={ql} P={ptok} waves={nw}")
        B.pa_decode(qd, kd, vd, td, ld, w.num_kv_heads, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len, kernel="mfma", waves_per_item=nw)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        check(got, ref, w, f"heavy block q_len={ql} P={ptok} waves={nw}", a=a)
