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
      result records a digest of the kernel's sources (--sources gemm or
      decode); bench.py reports the gate/up traffic only while the sources
      still match it.

  python3 -m int4_grouped_gemm_router_amd.profiling counters --dir DIR [--dir DIR ...] \
        --command ... --out FILE
      Mean value per dispatch of every counter collected by one or more
      `rocprofv3 --pmc ... -d DIR -o run` passes, per kernel of the layer (the
      ceiling measurement kernels are left out), with a few derived figures (matrix-core busy share, bf16 TFLOP/s from
      the MFMA op count, VALU instructions per MFMA, L2 hit rate).
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

# sources that define the grouped GEMM kernels' code, and the decode kernels'
GEMM_SOURCES = ["csrc/gemm.hip", "csrc/gemm_wide.hip", "csrc/kernels.h", "csrc/device.h", "csrc/layout.h"]
DECODE_SOURCES = ["csrc/decode.hip", "csrc/topk.h", "csrc/kernels.h", "csrc/device.h", "csrc/layout.h"]


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
        "sources": a.sources, "sources_sha256": sources_digest(a.sources),
        "commands": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


N_SIMDS = 256 * 4  # compute units x SIMDs of one MI355X
N_XCDS = 8


def counters(dirs, commands, out, match="moe::", skip="ceiling_"):
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    for d in dirs:
        seen = set()
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = r["Kernel_Name"]
            if match not in k or skip in k:  # the layer's kernels, not the measurement helpers
                continue
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            key = (d, r["Dispatch_Id"])
            if key not in seen:
                seen.add(key)
                durs[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    lines = ["# rocprofv3 hardware counters, mean per dispatch", "# commands:"]
    lines += [f"#   {c}" for c in commands]
    lines += ["# derived (MI355X: 1024 SIMDs in 8 XCDs; GRBM_GUI_ACTIVE reads the sum over the XCDs):",
              "#   mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (1024 * GRBM_GUI_ACTIVE / 8)",
              "#   bf16_tflops = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 / dispatch duration (counter run)",
              "#   valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA",
              "#   valu_issue = 4 * SQ_ACTIVE_INST_VALU / (1024 * GRBM_GUI_ACTIVE / 8)",
              "#   wave_wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES, l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS)", ""]
    for k in sorted(vals, key=lambda k: -max(durs[k]) if durs[k] else 0):
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        dur = sum(durs[k]) / len(durs[k])
        name = k if len(k) <= 70 else k[:67] + "..."
        lines.append(f"{name}  (mean dispatch {dur * 1e6:.1f} us in the counter runs)")
        for c in sorted(m):
            lines.append(f"    {c:<34s} {m[c]:>16.0f}")
        cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / N_XCDS
        der = []
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            der.append(f"mfma_busy {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMDS * cyc):.3f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m and dur > 0:
            der.append(f"bf16_tflops {512 * m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] / dur / 1e12:.1f}")
        if m.get("SQ_INSTS_MFMA"):
            der.append(f"valu_per_mfma {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f}")
        if cyc and "SQ_ACTIVE_INST_VALU" in m:
            der.append(f"valu_issue {4 * m['SQ_ACTIVE_INST_VALU'] / (N_SIMDS * cyc):.3f}")
        if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in m:
            der.append(f"wave_wait {m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}")
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m and m["TCC_HIT_sum"] + m["TCC_MISS_sum"] > 0:
            der.append(f"l2_hit {m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.3f}")
        if der:
            lines.append("    derived: " + ", ".join(der))
        lines.append("")
    text = "\n".join(lines)
    with open(out, "w") as f:
        f.write(text)
    print(text)


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
    t.add_argument("--sources", choices=["gemm", "decode"], default="gemm",
                   help="source set whose digest the summary records")
    c = sub.add_parser("counters")
    c.add_argument("--dir", action="append", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "traffic":
        a.sources = GEMM_SOURCES if a.sources == "gemm" else DECODE_SOURCES
    if a.cmd == "copy":
        run_copy()
    elif a.cmd == "kernel-stats":
        kernel_stats(a.dir, a.command, a.out)
    elif a.cmd == "counters":
        counters(a.dir, a.command, a.out)
    else:
        traffic(a)


if __name__ == "__main__":
    main(sys.argv[1:])
