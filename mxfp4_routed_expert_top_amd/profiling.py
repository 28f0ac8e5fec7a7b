"""Reading rocprofv3 output: per-kernel counter means and HBM traffic records.

HBM traffic of a kernel comes from two ``rocprofv3 --pmc`` passes over the
same program (``FETCH_SIZE``, then ``WRITE_SIZE``, both in KiB per
dispatch).  Each counter is scaled by what it reads for a plain kernel of
known size run in the same program (``bench.py --pmc-calibrate`` runs
``torch.bitwise_not`` over 1 GiB of int32 first: it reads 1 GiB and writes
1 GiB), so the factor is measured, not assumed.

A traffic record also stores a SHA-256 over the library's kernel sources;
``load_traffic`` returns None once any of them has changed, so a stale
measurement is never reported as current.

  python -m mxfp4_routed_expert_top_amd.profiling traffic \\
      --fetch <dir of the FETCH_SIZE pass> --write <dir of the WRITE_SIZE pass> \\
      --workload decode --out profiles/<name>.json
  python -m mxfp4_routed_expert_top_amd.profiling counters <dir> ...
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
CALIBRATION_KERNEL = "bitwise_not"
CALIBRATION_BYTES = 1 << 30      # read and written by the calibration kernel


def source_digest() -> str:
    """SHA-256 over every kernel source of the library (sorted by name)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def short_name(kernel: str) -> str:
    n = kernel.replace("void ", "").replace("(anonymous namespace)::", "")
    cut = n.find("(", 1)
    return n[:cut] if cut > 0 else n


def counter_means(directory: str) -> dict:
    """{kernel short name: {counter: (dispatches, mean value)}} over every
    counter_collection.csv under directory."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                agg[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: (len(v), sum(v) / len(v)) for c, v in cs.items()} for k, cs in agg.items()}


def _calibration(means: dict, counter: str) -> float:
    hits = [v[counter][1] for k, v in means.items() if CALIBRATION_KERNEL in k and counter in v]
    if len(hits) != 1:
        raise ValueError(f"expected one {CALIBRATION_KERNEL} dispatch with {counter}, found {len(hits)}")
    return CALIBRATION_BYTES / (hits[0] * 1024.0)


def traffic_record(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """Per-kernel HBM bytes per dispatch: counter KiB x 1024 x calibration factor."""
    fm, wm = counter_means(fetch_dir), counter_means(write_dir)
    ff, wf = _calibration(fm, "FETCH_SIZE"), _calibration(wm, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fm) & set(wm)):
        if CALIBRATION_KERNEL in k or "FETCH_SIZE" not in fm[k] or "WRITE_SIZE" not in wm[k]:
            continue
        n, fk = fm[k]["FETCH_SIZE"]
        _, wk = wm[k]["WRITE_SIZE"]
        kernels[k] = {"dispatches": n, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                      "fetch_bytes": round(fk * 1024 * ff), "write_bytes": round(wk * 1024 * wf),
                      "bytes": round(fk * 1024 * ff + wk * 1024 * wf)}
    cmd = (f"rocprofv3 --pmc {{counter}} -f csv -d <dir> -o p -- python -u <repo>/bench.py "
           f"--workload {workload} --no-cpu --steps 5 --warmup 2 --pmc-calibrate")
    return {"workload": workload, "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
            "commands": ["cd /tmp && export TMPDIR=/tmp", cmd.format(counter="FETCH_SIZE"),
                         cmd.format(counter="WRITE_SIZE"),
                         "python -m mxfp4_routed_expert_top_amd.profiling traffic --fetch <FETCH_SIZE dir> "
                         f"--write <WRITE_SIZE dir> --workload {workload} --out <record>"],
            "calibration": f"torch.bitwise_not over {CALIBRATION_BYTES} B of int32 "
                           f"(reads and writes {CALIBRATION_BYTES} B)",
            "source_sha256": source_digest(), "kernels": kernels}


def load_traffic(path: str, kernel: str):
    """HBM bytes per dispatch of kernel from a traffic record, or None when the
    record is missing, lacks the kernel, or the kernel sources changed since."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["bytes"]


def main(argv=None):
    p = argparse.ArgumentParser(prog="python -m mxfp4_routed_expert_top_amd.profiling")
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    a = p.parse_args(argv)
    if a.cmd == "traffic":
        rec = traffic_record(a.fetch, a.write, a.workload)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
    else:
        for d in a.dirs:
            print("##", d)
            for k, cs in sorted(counter_means(d).items()):
                print(k, {c: (n, round(v, 1)) for c, (n, v) in cs.items()})


if __name__ == "__main__":
    sys.exit(main())
