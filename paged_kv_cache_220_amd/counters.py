"""HBM traffic per partition-kernel launch from rocprofv3 counter runs.

Takes the counter CSVs of two ``rocprofv3 --pmc`` runs of ``bench.py --copy-probe MIB`` (one run
with FETCH_SIZE, one with WRITE_SIZE; both counters in KiB per dispatch) and writes the entry that
``bench.py`` reports as ``roofline.traffic``:

- the device copy of known size that ``--copy-probe`` dispatches first calibrates each counter
  (scale = bytes the copy really reads or writes / bytes the counter reports for it);
- the partition kernel's mean FETCH_SIZE and WRITE_SIZE over its dispatches, each times its scale,
  give the bytes per launch;
- the entry records a digest of the kernel's sources, so it goes stale (null in the bench line) as
  soon as the kernel changes.

Usage (on the host, after copying the two CSVs back)::

    python -m paged_kv_cache_220_amd.counters --fetch F.csv --write W.csv --workload c3 \\
        --partition-tokens 4096 --copy-mib 1024
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["pa_internal.h", "pa_device.h", "pa_api.hip", "pa_mfma.hip"]
VALU_KERNEL_SOURCES = ["pa_internal.h", "pa_device.h", "pa_api.hip", "pa_valu.hip"]
COPY_KERNEL = "copyBuffer"
PARTITION_KERNEL = "_partition"   # matrix-core (grid or work-list form) or vector partition kernel
REDUCE_KERNEL = "reduce_"   # the merge kernel in either form


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _csv_path(p):
    if os.path.isdir(p):
        hits = sorted(glob.glob(os.path.join(p, "**", "*counter_collection.csv"), recursive=True))
        if not hits:
            raise SystemExit(f"no *counter_collection.csv under {p}")
        return hits[0]
    return p


def read_counter(path, counter):
    """{kernel name: [value per dispatch]} for one counter (rows of one dispatch are summed)."""
    per_dispatch = defaultdict(float)
    names = {}
    with open(_csv_path(path), newline="") as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            d = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per_dispatch[d] += float(row["Counter_Value"])
            names[d] = row.get("Kernel_Name", "")
    out = defaultdict(list)
    for d in sorted(per_dispatch, key=lambda x: int(x)):
        out[names[d]].append(per_dispatch[d])
    return out


def _pick(per_kernel, needle):
    hits = {k: v for k, v in per_kernel.items() if needle in k}
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {sorted(hits)}")
    (name, vals), = hits.items()
    return name, vals


def build_entry(fetch, write, copy_bytes, algorithmic_bytes):
    # the probe's dispatches only: the runtime also launches small copies of its own
    probe = lambda v: [x for x in v if x >= 0.1 * copy_bytes / 1024.0]
    cf = probe(_pick(fetch, COPY_KERNEL)[1])
    cw = probe(_pick(write, COPY_KERNEL)[1])
    if not cf or not cw:
        raise SystemExit("no copy-probe dispatch of the stated size in the counter runs")
    kname, pf = _pick(fetch, PARTITION_KERNEL)
    _, pw = _pick(write, PARTITION_KERNEL)
    sources = VALU_KERNEL_SOURCES if "valu_partition" in kname else KERNEL_SOURCES
    mean = lambda v: sum(v) / len(v)
    fetch_scale = copy_bytes / 1024.0 / mean(cf)
    write_scale = copy_bytes / 1024.0 / mean(cw)
    traffic = (mean(pf) * fetch_scale + mean(pw) * write_scale) * 1024.0
    e = {
        "kernel_source_files": sources,
        "kernel_source_sha256": source_digest(sources),
        "kernel": kname,
        "fetch_kib_per_dispatch": round(mean(pf), 1),
        "write_kib_per_dispatch": round(mean(pw), 1),
        "copy_probe_bytes": copy_bytes,
        "copy_fetch_kib": round(mean(cf), 1),
        "copy_write_kib": round(mean(cw), 1),
        "fetch_scale": round(fetch_scale, 5),
        "write_scale": round(write_scale, 5),
        "traffic_bytes_per_launch": int(round(traffic)),
        "algorithmic_bytes_per_launch": int(algorithmic_bytes),
        "dispatches_averaged": min(len(pf), len(pw)),
    }
    try:
        _, rf = _pick(fetch, REDUCE_KERNEL)
        _, rw = _pick(write, REDUCE_KERNEL)
        e["reduce_kernel"] = {"fetch_kib": round(mean(rf), 1), "write_kib": round(mean(rw), 1)}
    except SystemExit:
        pass
    return e


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--fetch", required=True, help="counter CSV (or its directory) of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="counter CSV (or its directory) of the WRITE_SIZE run")
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--kv-dtype", default="")
    ap.add_argument("--q-len", type=int, default=1)
    ap.add_argument("--partition-tokens", type=int, required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    args = ap.parse_args(argv)

    sys.path.insert(0, ROOT)
    from paged_kv_cache_220_amd import accounting as A
    from paged_kv_cache_220_amd import workloads as W
    lens = W.batch_seq_lens(args.workload)
    _, hkv, d, _, kvd = W.batch_heads(args.workload, args.kv_dtype or None)
    alg = A.algorithmic_kv_bytes(lens, hkv, d, kvd)

    entry = build_entry(read_counter(args.fetch, "FETCH_SIZE"), read_counter(args.write, "WRITE_SIZE"),
                        args.copy_mib << 20, alg)
    batch = args.workload + (f"-{args.kv_dtype}" if args.kv_dtype else "") + (f"-q{args.q_len}" if args.q_len > 1 else "")
    prefix = "pa_valu_partition" if "valu_partition" in entry["kernel"] else "pa_mfma_partition"
    key = f"{prefix}:{batch}:{args.partition_tokens}"
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    t.setdefault("_about", "HBM bytes per partition-kernel launch from rocprofv3 --pmc FETCH_SIZE and "
                 "WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the same counter read "
                 "a device copy of known size as that size; valid while the listed sources hash to "
                 "kernel_source_sha256")
    t[key] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")
    print(json.dumps({key: entry}, indent=1))


if __name__ == "__main__":
    main()
