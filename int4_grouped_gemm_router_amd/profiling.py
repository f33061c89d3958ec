"""Helpers for the rocprofv3 summaries kept with the project.

Commands (run from the repository root):

  python3 -m int4_grouped_gemm_router_amd.profiling copy
      A plain device copy of 256 MiB, three times: the workload whose
      FETCH_SIZE / WRITE_SIZE readings calibrate those counters (the copy
      reads and writes exactly 256 MiB per dispatch). Needs a GPU.

  python3 -m int4_grouped_gemm_router_amd.profiling kernel-stats DIR --command CMD --out FILE
      Turns a `rocprofv3 --kernel-trace --stats -d DIR -o run` result into a
      short text table (calls, mean / min / max duration per kernel).

  python3 -m int4_grouped_gemm_router_amd.profiling traffic --fetch DIR --write DIR \
        --copy-fetch DIR --copy-write DIR --kernel NAME --grid N --command ... --out FILE
      Mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of one kernel, scaled
      by the factors the copy dispatches give, as HBM bytes per launch. The
      result records a digest of the kernel's sources; bench.py reports the
      traffic only while the sources still match it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20

# sources that define the grouped GEMM kernels' code
GEMM_SOURCES = ["csrc/gemm.hip", "csrc/kernels.h", "csrc/device.h", "csrc/layout.h"]


def sources_digest(files=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def run_copy():
    import torch
    x = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3", flush=True)


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def kernel_stats(d, command, out):
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
             f"# {'kernel':<58s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for r in rows:
        name = r["Name"]
        if len(name) > 58:
            name = name[:55] + "..."
        lines.append(f"  {name:<58s} {int(r['Calls']):>6d} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                     f"{float(r['Percentage']):>7.2f}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    print(text)


def _counter_means(d, counter):
    """Mean counter value per (kernel name, grid size) over its dispatches."""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        acc[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _copy_factor(d, counter):
    m = _counter_means(d, counter)
    vals = [v for (name, _), (v, _) in m.items() if "copyBuffer" in name]
    if not vals:
        raise RuntimeError(f"no copy dispatch with {counter} under {d}")
    kib = max(vals)
    return (COPY_BYTES / 1024.0) / kib, kib


def traffic(a):
    fetch = _counter_means(a.fetch, "FETCH_SIZE")
    write = _counter_means(a.write, "WRITE_SIZE")
    fk = [(k, v) for k, v in fetch.items() if a.kernel in k[0] and (a.grid is None or k[1] == a.grid)]
    wk = [(k, v) for k, v in write.items() if a.kernel in k[0] and (a.grid is None or k[1] == a.grid)]
    if len(fk) != 1 or len(wk) != 1:
        raise RuntimeError(f"kernel {a.kernel!r} grid {a.grid}: matched {fk} / {wk}")
    ff, fcopy = _copy_factor(a.copy_fetch, "FETCH_SIZE")
    wf, wcopy = _copy_factor(a.copy_write, "WRITE_SIZE")
    (key, (fkib, nf)), (_, (wkib, nw)) = fk[0], wk[0]
    res = {
        "kernel": key[0], "grid_size": key[1], "dispatches": [nf, nw],
        "fetch_kib_per_dispatch": fkib, "write_kib_per_dispatch": wkib,
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
        "fetch_scale": ff, "write_scale": wf,
        "hbm_bytes_per_launch": fkib * 1024 * ff + wkib * 1024 * wf,
        "sources": GEMM_SOURCES, "sources_sha256": sources_digest(),
        "commands": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("copy")
    k = sub.add_parser("kernel-stats")
    k.add_argument("dir")
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "out"):
        t.add_argument("--" + n.replace("_", "-"), dest=n, required=True)
    t.add_argument("--grid", type=int, default=None)
    t.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        run_copy()
    elif a.cmd == "kernel-stats":
        kernel_stats(a.dir, a.command, a.out)
    else:
        traffic(a)


if __name__ == "__main__":
    main(sys.argv[1:])
