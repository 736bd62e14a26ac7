"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Small copies of every decode batch, and every batch at full size in the
launch configuration the benchmark times, are compared element by element
over the whole output. Bitwise checks: repeated runs, relabelled
physical blocks and NaN-poisoned unread memory must not change one bit.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import abs_attention_multi, check, log, oracle_full, run_gpu, upload
from oracle import pa_oracle as O
from paged_kv_cache_220_amd import binding as B
from paged_kv_cache_220_amd import workloads as W

pytestmark = pytest.mark.gpu


def kernels_for(w):
    """Kernels that take this batch (planning only reads the scale pointers' presence)."""
    ks = []
    sc = dict(k_block_scales=4096, v_block_scales=8192) if w.k_block_scales is not None else {}
    try:
        B.plan(B.PaDims(num_seqs=w.num_seqs, num_heads=w.num_heads, head_dim=w.head_dim, num_blocks=w.num_blocks,
                        block_size=w.block_size, max_blocks_per_seq=w.max_blocks_per_seq,
                        q_dtype=B._KV_NAMES[w.q_dtype], kv_dtype=B._KV_NAMES[w.kv_dtype], k_scale=1.0, v_scale=1.0,
                        max_seq_len=0, partition_tokens=0, kernel=B.KERNELS["valu"], **sc), w.num_kv_heads)
        ks.append("valu")
    except B.PagedAttentionError:
        pass
    dims = B.PaDims(num_seqs=w.num_seqs, num_heads=w.num_heads, head_dim=w.head_dim, num_blocks=w.num_blocks,
                    block_size=w.block_size, max_blocks_per_seq=w.max_blocks_per_seq,
                    q_dtype=B._KV_NAMES[w.q_dtype], kv_dtype=B._KV_NAMES[w.kv_dtype], k_scale=1.0, v_scale=1.0,
                    max_seq_len=0, partition_tokens=0, kernel=B.KERNELS["mfma"], **sc)
    try:
        B.plan(dims, w.num_kv_heads)
        ks.append("mfma")
    except B.PagedAttentionError:
        pass
    return ks


SMALL = [("c1", {}), ("c2", dict(num_seqs=12)), ("c3", dict(num_seqs=2, seq_len=3000)),
         ("c4", dict(num_seqs=20, seq_len=5000)), ("c5", dict(num_seqs=4, seq_len=2100)),
         ("c5", dict(num_seqs=4, seq_len=2100, kv_dtype="e4m3")),
         ("c2", dict(num_seqs=12, kv_dtype="int4")), ("c3", dict(num_seqs=2, seq_len=3000, kv_dtype="int4")),
         ("c4", dict(num_seqs=20, seq_len=5000, kv_dtype="int4"))]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] + s[1].get("kv_dtype", "") for s in SMALL])
@pytest.mark.parametrize("ptok", [0, 64, 256])
def test_small_batches(name, kw, ptok):
    w = W.make_workload(name, **kw)
    ref = oracle_full(w)
    dev = upload(w)
    for kern in kernels_for(w):
        log(f"case {name}{kw} kernel={kern} partition_tokens={ptok}")
        got = run_gpu(w, dev, kernel=kern, partition_tokens=ptok)
        check(got, ref, w, f"{name} {kern} P={ptok}")


EDGE = [
    ("bf16 G8 D128", dict(S=9, H=16, Hkv=2, D=128, seq_lens=[0, 1, 15, 16, 17, 63, 64, 65, 200])),
    ("bf16 G1 D128", dict(S=4, H=4, Hkv=4, D=128, seq_lens=[1, 33, 0, 129])),
    ("bf16 G2 D64", dict(S=3, H=8, Hkv=4, D=64, seq_lens=[5, 70, 300])),
    ("bf16 G4 D128", dict(S=3, H=8, Hkv=2, D=128, seq_lens=[31, 97, 513])),
    ("bf16 G16 D128", dict(S=3, H=32, Hkv=2, D=128, seq_lens=[2, 100, 700])),
    ("bf16 G3 D128", dict(S=3, H=6, Hkv=2, D=128, seq_lens=[7, 64, 450])),
    ("e5m2 G5 D128", dict(S=2, H=10, Hkv=2, D=128, seq_lens=[30, 333], kv_dtype="e5m2")),
    ("f32 G1 D64", dict(S=5, H=2, Hkv=2, D=64, seq_lens=[0, 1, 16, 17, 400], q_dtype="f32", kv_dtype="f32")),
    ("f32 G8 D128", dict(S=3, H=16, Hkv=2, D=128, seq_lens=[3, 64, 190], q_dtype="f32", kv_dtype="f32")),
    ("e5m2 G8 D128", dict(S=5, H=16, Hkv=2, D=128, seq_lens=[1, 16, 17, 64, 333], kv_dtype="e5m2")),
    ("e5m2 G4 D64", dict(S=3, H=8, Hkv=2, D=64, seq_lens=[9, 80, 260], kv_dtype="e5m2")),
    ("e4m3 G8 D128", dict(S=5, H=16, Hkv=2, D=128, seq_lens=[1, 16, 17, 64, 333], kv_dtype="e4m3")),
    ("int4 G8 D128", dict(S=9, H=16, Hkv=2, D=128, seq_lens=[0, 1, 15, 16, 17, 63, 64, 65, 333], kv_dtype="int4")),
    ("int4 G3 D128", dict(S=3, H=6, Hkv=2, D=128, seq_lens=[7, 64, 450], kv_dtype="int4")),
    ("e4m3 G4 D64", dict(S=3, H=8, Hkv=2, D=64, seq_lens=[9, 80, 260], kv_dtype="e4m3")),
]


@pytest.mark.parametrize("label,kw", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("ptok", [0, 64])
def test_edge_shapes(label, kw, ptok):
    w = W.random_edge_workload(len(label) + ptok, **kw)
    ref = oracle_full(w)
    dev = upload(w)
    for kern in kernels_for(w):
        log(f"case edge {label} kernel={kern} partition_tokens={ptok}")
        got = run_gpu(w, dev, kernel=kern, partition_tokens=ptok)
        check(got, ref, w, f"{label} {kern} P={ptok}")
        zero = w.seq_lens == 0
        assert np.all(got[zero] == 0)


def test_library_workspace_path_matches_caller_workspace():
    w = W.make_workload("c3", num_seqs=2, seq_len=2000)
    dev = upload(w)
    for kern in kernels_for(w):
        a = run_gpu(w, dev, kernel=kern, partition_tokens=128, use_workspace=True)
        b = run_gpu(w, dev, kernel=kern, partition_tokens=128, use_workspace=False)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name,kw", [("c1", {}), ("c2", dict(num_seqs=8)), ("c4", dict(num_seqs=12, seq_len=3000)),
                                     ("c5", dict(num_seqs=3, seq_len=1500)),
                                     ("c5", dict(num_seqs=3, seq_len=1500, kv_dtype="e4m3")),
                                     ("c4", dict(num_seqs=12, seq_len=3000, kv_dtype="int4"))])
def test_bitwise_repeat_relabel_poison(name, kw):
    w = W.make_workload(name, **kw)
    wp = W.permute_pool(w, 5)
    wn = W.make_workload(name, poison=True, **kw)
    for kern in kernels_for(w):
        log(f"case bitwise {name} kernel={kern}")
        a = run_gpu(w, kernel=kern, partition_tokens=128)
        b = run_gpu(w, kernel=kern, partition_tokens=128)
        c = run_gpu(wp, kernel=kern, partition_tokens=128)
        d = run_gpu(wn, kernel=kern, partition_tokens=128)
        assert np.array_equal(a, b), "repeat"
        assert np.array_equal(a, c), "relabelled blocks"
        assert np.array_equal(a, d), "poisoned unread memory"


def test_special_values_single_token_and_zero_query():
    w = W.random_edge_workload(7, S=3, H=16, Hkv=2, D=128, seq_lens=[1, 1, 1])
    dev = upload(w)
    for kern in kernels_for(w):
        got = run_gpu(w, dev, kernel=kern)
        # one token: softmax weight exactly 1, output is that token's V row (bf16 values, exact)
        for s in range(3):
            b = w.block_tables[s, 0]
            for h in range(16):
                vrow = (w.v_cache[b, h // 8, :, 0].astype(np.uint32) << 16).view(np.float32)
                assert np.array_equal(got[s, h], vrow.astype(np.float64))
    w2 = W.make_workload("c2", num_seqs=4)
    w2.q[:] = 0
    ref = oracle_full(w2)
    for kern in kernels_for(w2):
        check(run_gpu(w2, kernel=kern), ref, w2, f"q=0 {kern}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "e5m2", "int4"])
@pytest.mark.parametrize("boost", [32.0, 1024.0])
def test_peaked_softmax(kv_dtype, boost):
    """Large scores: the scale times 32 (scores of tens) or 1024 (scores of
    thousands, where every weight but the largest underflows to 0 and the
    output is one token's V row). The running max keeps every exponent <= 0."""
    w = W.make_workload("c2", num_seqs=6, kv_dtype=None if kv_dtype == "bf16" else kv_dtype)
    w.scale = np.float32(w.scale * np.float32(boost))      # a power of two: exact
    ref = oracle_full(w)
    dev = upload(w)
    for kern in kernels_for(w):
        for ptok in (0, 64):
            got = run_gpu(w, dev, kernel=kern, partition_tokens=ptok)
            check(got, ref, w, f"peaked x{boost:g} {kv_dtype} {kern} P={ptok}")


# ---------------------------------------------------------------- full size --

FULL = ["c2", "c3", "c4", "c5"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """The batch at full size, in the launch configuration the benchmark times
    (default plan), every sequence and head against the oracle."""
    w = W.make_workload(name)
    dev = upload(w)
    log(f"case full {name}: oracle over all {w.num_seqs} sequences")
    ref = oracle_full(w)
    for kern in kernels_for(w):
        log(f"case full {name} kernel={kern} (default plan)")
        got = run_gpu(w, dev, kernel=kern)
        check(got, ref, w, f"full {name} {kern}")
        del got
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["bf16", "e5m2"])
def test_one_sequence_of_128k_tokens(kv_dtype):
    """A context longer than the batches: one sequence of 131,072 tokens (the
    page's 128K-context example). The default plan shortens partitions to put
    enough waves on the chip (hundreds of partitions, so the merge takes its
    many-partition form); every head is checked against the oracle."""
    w = W.make_workload("c3", num_seqs=1, seq_len=131072, kv_dtype=None if kv_dtype == "bf16" else kv_dtype)
    dev = upload(w)
    d = B.make_dims(dev["q"], dev["k"], dev["tables"], max_seq_len=w.max_seq_len)
    plan = B.plan(d, w.num_kv_heads)
    log(f"case 128k {kv_dtype}: plan {plan}")
    assert plan["max_partitions"] > 8
    ref = oracle_full(w)
    for kern in kernels_for(w):
        got = run_gpu(w, dev, kernel=kern)
        check(got, ref, w, f"128k {kv_dtype} {kern}")
    del dev
    torch.cuda.empty_cache()


# ------------------------------------------------------------ queue schedule --

QUEUE = [("c4", dict(num_seqs=40, seq_len=6000), 0), ("c4", dict(num_seqs=40, seq_len=6000), 512),
         ("c2", dict(num_seqs=16), 128), ("c5", dict(num_seqs=5, seq_len=2500), 1024),
         ("c3", dict(num_seqs=2, seq_len=4100), 2048)]


@pytest.mark.parametrize("name,kw,ptok", QUEUE, ids=[f"{q[0]}-P{q[2]}" for q in QUEUE])
def test_queue_schedule_matches_grid(name, kw, ptok):
    """With the same waves per item, the work-list schedule computes every
    item exactly as the grid does."""
    w = W.make_workload(name, **kw)
    dev = upload(w)
    ref = oracle_full(w)
    for nw in (1, 4):
        log(f"case queue {name}{kw} P={ptok} waves={nw}")
        g = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, schedule="grid", waves_per_item=nw)
        q = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, schedule="queue", waves_per_item=nw)
        assert np.array_equal(g, q)
        check(q, ref, w, f"queue {name} P={ptok} waves={nw}")


# ---------------------------------------------------------- waves per item --

WAVES = [("c2", dict(num_seqs=12), 512), ("c3", dict(num_seqs=2, seq_len=4100), 0),
         ("c5", dict(num_seqs=6, seq_len=1900), 1024), ("c5", dict(num_seqs=4, seq_len=700, kv_dtype="e4m3"), 0),
         ("c4", dict(num_seqs=30, seq_len=3000), 256), ("c5", dict(num_seqs=4, seq_len=900, kv_dtype="int4"), 0)]


@pytest.mark.parametrize("name,kw,ptok", WAVES, ids=[f"{c[0]}{c[1].get('kv_dtype', '')}-P{c[2]}" for c in WAVES])
def test_waves_per_item(name, kw, ptok):
    """Items split over 1 to 4 waves (tiles strided over the waves, states
    merged in LDS) all match the oracle, on both schedules."""
    w = W.make_workload(name, **kw)
    dev = upload(w)
    ref = oracle_full(w)
    for nw in (1, 2, 3, 4):
        for sched in ("grid", "queue"):
            log(f"case waves {name}{kw} P={ptok} waves={nw} {sched}")
            got = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, schedule=sched, waves_per_item=nw)
            check(got, ref, w, f"waves {name} P={ptok} waves={nw} {sched}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "e5m2", "e4m3", "int4"])
def test_waves_per_item_edge_lengths(kv_dtype):
    """Waves past the end of a short item contribute an empty state; partial
    last tiles and blocks past the partition end are masked (fp8 K through LDS too)."""
    w = W.random_edge_workload(41, S=10, H=16, Hkv=2, D=128, kv_dtype=kv_dtype,
                               seq_lens=[0, 1, 15, 16, 17, 63, 64, 65, 129, 300])
    ref = oracle_full(w)
    dev = upload(w)
    for nw in (1, 2, 3, 4):
        for ptok in (64, 128, 256):
            got = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, waves_per_item=nw)
            check(got, ref, w, f"waves edge P={ptok} waves={nw}")
            assert np.all(got[0] == 0)


def test_queue_schedule_edge_lengths():
    w = W.random_edge_workload(31, S=9, H=16, Hkv=2, D=128, seq_lens=[0, 1, 15, 16, 17, 63, 64, 65, 900])
    ref = oracle_full(w)
    dev = upload(w)
    for ptok in (64, 128):
        got = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, schedule="queue")
        check(got, ref, w, f"queue edge P={ptok}")
        assert np.all(got[0] == 0)



def test_queue_schedule_many_sequences():
    """More sequences than the plan kernel has threads, several times over
    (5,000: each thread counts and places 4 or 5 of them), lengths 0 to 300
    with many zeros; the work list must still cover every item exactly once."""
    rng = np.random.default_rng(5000)
    lens = rng.integers(0, 301, 5000)
    lens[rng.random(5000) < 0.1] = 0
    w = W.random_edge_workload(32, S=5000, H=8, Hkv=1, D=128, seq_lens=lens.tolist())
    ref = oracle_full(w)
    dev = upload(w)
    for ptok in (64, 128):
        got = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, schedule="queue")
        check(got, ref, w, f"queue 5000 seqs P={ptok}")
        assert np.all(got[lens == 0] == 0)


@pytest.mark.parametrize("kv_dtype", ["e5m2", "e4m3"])
def test_every_fp8_code_decodes_exactly(kv_dtype):
    """One-token sequences return their V row; two sequences cover all 256 codes.

    The output is bf16, and every finite fp8 value is exact in bf16, so each
    output element must equal the oracle's decoding of its code; non-finite
    codes must give non-finite outputs."""
    w = W.random_edge_workload(5, S=2, H=8, Hkv=1, D=128, seq_lens=[1, 1], kv_dtype=kv_dtype)
    codes = np.arange(256, dtype=np.uint8)
    for s in range(2):
        w.v_cache[w.block_tables[s, 0], 0, :, 0] = codes[128 * s:128 * (s + 1)]
        w.k_cache[w.block_tables[s, 0], 0, :, 0] = 0x3C if kv_dtype == "e5m2" else 0x38     # finite keys
    dev = upload(w)
    want = O.decode_bits(codes, kv_dtype).reshape(2, 128)
    for kern in kernels_for(w):
        got = run_gpu(w, dev, kernel=kern)
        for s in range(2):
            for h in range(8):
                fin = np.isfinite(want[s])
                assert np.array_equal(got[s, h][fin], want[s][fin]), (kern, s)
                assert not np.isfinite(got[s, h][~fin]).any(), (kern, s)


# ------------------------------------------------------------- int4 / scales --

def test_every_int4_code_decodes_exactly():
    """One-token sequences return their V row: code * v_block_scale, with power-of-two
    scales exact in bf16. Rows hold all 16 codes; K codes and scales vary too."""
    S, H, Hkv, D = 16, 16, 2, 128
    w = W.random_edge_workload(21, S=S, H=H, Hkv=Hkv, D=D, seq_lens=[1] * S, kv_dtype="int4")
    rng = np.random.default_rng(22)
    codes = (np.arange(D)[None, None, :] + np.arange(S)[:, None, None] + np.arange(Hkv)[None, :, None]) % 16 - 8
    for s_ in range(S):
        b = int(w.block_tables[s_, 0])
        for g in range(Hkv):
            row = O.int4_unpack(w.v_cache[b, g])                     # [D, 16]
            row[:, 0] = codes[s_, g]
            w.v_cache[b, g] = O.int4_pack(row)
    w.v_block_scales[:] = np.exp2(rng.integers(-4, 3, w.v_block_scales.shape)).astype(np.float32)
    got = run_gpu(w)
    for s_ in range(S):
        b = int(w.block_tables[s_, 0])
        for h in range(H):
            g = h // (H // Hkv)
            assert np.array_equal(got[s_, h], codes[s_, g].astype(np.float64) * float(w.v_block_scales[b, g]))


@pytest.mark.parametrize("kv_dtype", ["e5m2", "e4m3"])
def test_fp8_with_block_scales(kv_dtype):
    """fp8 caches with per-(block, KV head) scales on top of the per-tensor ones."""
    w = W.make_workload("c5", num_seqs=6, seq_len=1300, kv_dtype=kv_dtype)
    rng = np.random.default_rng(23)
    w.k_block_scales = np.exp2(rng.uniform(-2, 2, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
    w.v_block_scales = np.exp2(rng.uniform(-2, 2, (w.num_blocks, w.num_kv_heads))).astype(np.float32)
    w.k_scale, w.v_scale = np.float32(0.75), np.float32(1.25)
    ref = oracle_full(w)
    dev = upload(w)
    for ptok, nw in ((0, 0), (256, 2), (64, 4)):
        log(f"case fp8 block scales {kv_dtype} P={ptok} waves={nw}")
        check(run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, waves_per_item=nw), ref, w,
              f"{kv_dtype} block scales P={ptok}")


def test_int4_full_size():
    """The int4 form of the long-context batch at full size, every sequence."""
    w = W.make_workload("c3", kv_dtype="int4")
    log("case full c3 int4: oracle over all sequences")
    ref = oracle_full(w)
    dev = upload(w)
    log("case full c3 int4 (default plan)")
    check(run_gpu(w, dev), ref, w, "full c3 int4")
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["e5m2", "e4m3", "int4"])
def test_one_part_decode_every_block_counted_once(kv_dtype):
    """fp8 and int4 decode feed each weight to PV as one binary16 value, so
    their outputs are held to 2^-7 |ref| + 2^-10 a + 1e-4 (a: the attention
    over |V|); on sequences of several thousand tokens that lets one ordinary
    skipped block pass. Here one block per sequence holds V = 32 under
    near-uniform weights (q x 2^-20): the first block, one mid-partition, the
    first of the second 4096-token partition, and the last, partly filled one
    (int4: codes 4 at block scale 8). Skipping or repeating it moves the output
    by about 32 x its tokens / L, several times the gate."""
    lens = [9000, 8200, 6000, 4101]
    w = W.random_edge_workload(97, S=len(lens), H=64, Hkv=8, D=128, seq_lens=lens, kv_dtype=kv_dtype)
    heavy = [0, 100, 256, (lens[3] - 1) // 16]
    for s, b in enumerate(heavy):
        blk = int(w.block_tables[s, b])
        if kv_dtype == "int4":
            w.v_cache[blk] = O.int4_pack(np.full(w.v_cache.shape[1:3] + (16,), 4, np.int8))
            w.v_block_scales[blk] = 8.0
        else:
            w.v_cache[blk] = W.to_storage(np.full(w.v_cache.shape[1:], 32.0, np.float32), kv_dtype)
    qf = (w.q.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** -20)
    w.q = W.to_storage(qf, "bf16")
    ref = oracle_full(w)
    a = abs_attention_multi(w.q[:, None], w)[:, 0]
    ntok = [min(16, lens[s] - 16 * b) for s, b in enumerate(heavy)]
    gate = 2.0 ** -7 * np.abs(ref) + 2.0 ** -10 * a + 1e-4
    for s in range(w.num_seqs):
        assert gate[s].max() < 0.25 * 32.0 * ntok[s] / lens[s], f"sequence {s}: gate too loose"
    dev = upload(w)
    for ptok, nw, sched in ((0, 0, "auto"), (4096, 0, "grid"), (512, 2, "grid"), (1024, 3, "queue")):
        log(f"case one-part heavy block {kv_dtype} P={ptok} waves={nw} {sched}")
        got = run_gpu(w, dev, kernel="mfma", partition_tokens=ptok, waves_per_item=nw, schedule=sched)
        check(got, ref, w, f"one-part heavy block {kv_dtype} P={ptok} waves={nw} {sched}", a=a)
