"""Host logic that turns rocprofv3 counter CSVs into HBM bytes per launch (no GPU)."""

import csv

import numpy as np
import pytest

from paged_kv_cache_220_amd import counters as C
from paged_kv_cache_220_amd import workloads as W

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))


def test_calibrated_traffic_from_two_counter_runs(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    part = "void pa::mfma_partition_kernel<1, 1, 2, true, false, 0>(pa::Args, int)"
    red = "void pa::reduce_kernel<1>(pa::Args)"
    # the counter reads the 1 MiB copy as half its reads and all its writes
    fetch_rows = [(1, 1, copy, "FETCH_SIZE", 512.0), (2, 2, copy, "FETCH_SIZE", 512.0),
                  # one dispatch reported over two rows (summed), another over one
                  (3, 3, part, "FETCH_SIZE", 1000.0), (3, 3, part, "FETCH_SIZE", 1000.0),
                  (4, 4, red, "FETCH_SIZE", 10.0), (5, 5, part, "FETCH_SIZE", 2000.0),
                  (6, 6, copy, "FETCH_SIZE", 2.5)]  # a small runtime copy, not the probe
    write_rows = [(1, 1, copy, "WRITE_SIZE", 1024.0), (2, 2, copy, "WRITE_SIZE", 1024.0),
                  (3, 3, part, "WRITE_SIZE", 8.0), (4, 4, red, "WRITE_SIZE", 2.0),
                  (5, 5, part, "WRITE_SIZE", 8.0), (6, 6, copy, "WRITE_SIZE", 0.0625)]
    f, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(f, fetch_rows)
    _write_csv(wr, write_rows)
    e = C.build_entry(C.read_counter(str(f), "FETCH_SIZE"), C.read_counter(str(wr), "WRITE_SIZE"),
                      1 << 20, 4 << 20)
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["fetch_kib_per_dispatch"] == 2000.0 and e["write_kib_per_dispatch"] == 8.0
    assert e["traffic_bytes_per_launch"] == (2000 * 2 + 8) * 1024
    assert e["kernel"] == part and e["dispatches_averaged"] == 2
    assert e["reduce_kernel"] == {"fetch_kib": 10.0, "write_kib": 2.0}
    assert e["kernel_source_sha256"] == C.source_digest(C.KERNEL_SOURCES)


def test_ambiguous_kernel_match_is_an_error(tmp_path):
    rows = [(1, 1, "copyBuffer", "FETCH_SIZE", 1024.0), (2, 2, "mfma_partition_kernel<1>", "FETCH_SIZE", 1.0),
            (3, 3, "mfma_partition_kernel<2>", "FETCH_SIZE", 1.0)]
    f = tmp_path / "f.csv"
    _write_csv(f, rows)
    per = C.read_counter(str(f), "FETCH_SIZE")
    with pytest.raises(SystemExit):
        C.build_entry(per, per, 1 << 20, 1)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_batch_seq_lens_are_the_generated_ones(name):
    np.testing.assert_array_equal(W.batch_seq_lens(name), W.make_workload(name).seq_lens)
