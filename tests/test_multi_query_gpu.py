"""GPU parity of paged attention with several query positions per sequence
(speculative-decode verification, chunked prefill) against the oracle."""

import numpy as np
import pytest
import torch

from gpu_helpers import check, log
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
    qd = _dev(q, "bf16")
    out = torch.empty_like(qd)
    log(f"case multi-query {name}{kw} q_len={ql} P={ptok}")
    B.pa_decode(qd, _dev(w.k_cache, w.kv_dtype), _dev(w.v_cache, w.kv_dtype), torch.from_numpy(w.block_tables).cuda(),
                torch.from_numpy(w.seq_lens).cuda(), w.num_kv_heads, float(w.scale), out, partition_tokens=ptok,
                max_seq_len=w.max_seq_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    check(got, ref, w, f"multi-query {name} q_len={ql} P={ptok}")


@pytest.mark.parametrize("ql", [2, 4])
def test_multi_query_two_waves_per_item(ql):
    w = W.make_workload("c5", num_seqs=3, seq_len=2500)
    rng = np.random.default_rng([ql, 77])
    q = W.to_storage(rng.standard_normal((w.num_seqs, ql, w.num_heads, w.head_dim), dtype=np.float32), "bf16")
    ref = O.paged_attention_multi(q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.num_kv_heads, w.scale,
                                  "bf16", w.kv_dtype)
    qd = _dev(q, "bf16")
    for ptok in (0, 256):
        out = torch.empty_like(qd)
        log(f"case multi-query two waves q_len={ql} P={ptok}")
        B.pa_decode(qd, _dev(w.k_cache, w.kv_dtype), _dev(w.v_cache, w.kv_dtype),
                    torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.seq_lens).cuda(), w.num_kv_heads,
                    float(w.scale), out, partition_tokens=ptok, max_seq_len=w.max_seq_len, kernel="mfma",
                    waves_per_item=2)
        torch.cuda.synchronize()
        check(out.float().cpu().numpy().astype(np.float64), ref, w, f"multi-query 2 waves q_len={ql} P={ptok}")


def test_query_window_longer_than_sequence():
    """Early queries of a sequence shorter than the window see no token: zero rows."""
    w = W.random_edge_workload(3, S=4, H=16, Hkv=2, D=128, seq_lens=[1, 3, 70, 0])
    ql = 4
    rng = np.random.default_rng(8)
    q = W.to_storage(rng.standard_normal((4, ql, 16, 128), dtype=np.float32), "bf16")
    ref = O.paged_attention_multi(q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, 2, w.scale, "bf16", "bf16")
    for ptok in (0, 64):
        qd = _dev(q, "bf16")
        out = torch.full_like(qd, float("nan"))
        B.pa_decode(qd, _dev(w.k_cache, "bf16"), _dev(w.v_cache, "bf16"), torch.from_numpy(w.block_tables).cuda(),
                    torch.from_numpy(w.seq_lens).cuda(), 2, float(w.scale), out, partition_tokens=ptok,
                    max_seq_len=w.max_seq_len)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.all(got[0, :3] == 0) and np.all(got[1, :1] == 0) and np.all(got[3] == 0)
        check(got, ref, w, f"short window P={ptok}")
