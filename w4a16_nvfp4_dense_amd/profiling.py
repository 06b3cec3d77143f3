"""Summaries of rocprofv3 output for the library's kernels.

    python -m w4a16_nvfp4_dense_amd.profiling stats    TRACE_DIR  > summary.txt
    python -m w4a16_nvfp4_dense_amd.profiling traffic  FETCH_DIR WRITE_DIR KERNEL_SUBSTR OUT.json [SRC ...]
    python -m w4a16_nvfp4_dense_amd.profiling counters PMC_DIR [PMC_DIR ...]  > summary.md

``stats`` reads the ``*_kernel_stats.csv`` of a ``rocprofv3 --kernel-trace
--stats --output-format csv`` run. ``traffic`` reads two ``rocprofv3 --pmc``
runs (``FETCH_SIZE``, then ``WRITE_SIZE``, both in KiB per dispatch) of
``bench.py --calibrate-copy``: the 64 MiB device copy in that run is the
reference that scales each counter to bytes (on MI355X ``FETCH_SIZE`` reads
about half the copied bytes, ``WRITE_SIZE`` all of them). The JSON records a
digest of the measured kernel's source files (``SRC``, names under csrc/;
all of csrc/ by default), so ``bench.py`` only reports the traffic while
those sources are the ones that were measured. ``counters`` prints, for every
kernel of one or more ``rocprofv3 --pmc`` runs, the median over its
dispatches of each counter (summed over the counter's instances).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from typing import Dict, List

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
COPY_BYTES = 64 << 20  # the calibration copy of bench.py --calibrate-copy


def source_digest(files=None) -> str:
    """sha256 over kernel sources in name order: the named files of csrc/,
    or all of csrc/."""
    paths = (sorted(os.path.join(CSRC, f) for f in files) if files
             else sorted(glob.glob(os.path.join(CSRC, "*"))))
    h = hashlib.sha256()
    for path in paths:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _one(pattern: str) -> str:
    found = sorted(glob.glob(pattern, recursive=True))
    if not found:
        raise FileNotFoundError(pattern)
    return found[0]


def short_name(name: str) -> str:
    """A kernel's name without its parameter list (and without the
    anonymous-namespace qualifier, which would otherwise be cut at its own
    parenthesis)."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def stats_summary(trace_dir: str, top: int = 8) -> str:
    path = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    out = ["kernel | calls | average us | min us | max us | share %", "---|---|---|---|---|---"]
    for r in rows[:top]:
        name = short_name(r["Name"]) if "ffn::" in r["Name"] else r["Name"].replace("void ", "")[:60]
        out.append(f"{name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                   f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f}")
    return "\n".join(out)


def _counter_rows(run_dir: str, counter: str) -> List[dict]:
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]


def _per_dispatch(rows: List[dict]) -> Dict[int, dict]:
    out: Dict[int, dict] = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        e = out.setdefault(d, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "value": 0.0})
        e["value"] += float(r["Counter_Value"])
    return out


def counter_bytes(run_dir: str, counter: str, kernel_substr: str) -> dict:
    """Median KiB per dispatch of `counter` for the matching kernel, and the
    same counter for the calibration copy (the largest copy kernel)."""
    disp = _per_dispatch(_counter_rows(run_dir, counter))
    ker = [e["value"] for e in disp.values() if kernel_substr in e["name"]]
    copies = [e["value"] for e in disp.values()
              if ("copyBuffer" in e["name"] or "copy" in e["name"].lower()) and e["grid"] >= 65536]
    if not ker or not copies:
        raise ValueError(f"no dispatches for {kernel_substr!r} or no calibration copy in {run_dir}")
    return {"kernel_kib": statistics.median(ker), "copy_kib": max(copies), "n": len(ker)}


def traffic(fetch_dir: str, write_dir: str, kernel_substr: str, files=None) -> dict:
    f = counter_bytes(fetch_dir, "FETCH_SIZE", kernel_substr)
    w = counter_bytes(write_dir, "WRITE_SIZE", kernel_substr)
    f_scale = COPY_BYTES / (f["copy_kib"] * 1024.0)
    w_scale = COPY_BYTES / (w["copy_kib"] * 1024.0)
    fetch_b = f["kernel_kib"] * 1024.0 * f_scale
    write_b = w["kernel_kib"] * 1024.0 * w_scale
    return {
        "kernel": kernel_substr,
        "fetch_kib_raw": f["kernel_kib"], "write_kib_raw": w["kernel_kib"],
        "copy_fetch_kib_raw": f["copy_kib"], "copy_write_kib_raw": w["copy_kib"],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "fetch_bytes": fetch_b, "write_bytes": write_b, "bytes": fetch_b + write_b,
        "dispatches": f["n"],
        "source_files": sorted(files) if files else None,
        "source_digest": source_digest(files),
    }


def counters_summary(run_dirs: List[str]) -> str:
    """Markdown table: per kernel, the median over its dispatches of every
    counter collected in the runs (each summed over its instances)."""
    table: Dict[str, Dict[str, float]] = {}
    calls: Dict[str, int] = {}
    for d in run_dirs:
        path = _one(os.path.join(d, "**", "*counter_collection.csv"))
        per: Dict[tuple, float] = {}
        names: Dict[int, str] = {}
        for r in csv.DictReader(open(path)):
            key = (int(r["Dispatch_Id"]), r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
        byk: Dict[str, Dict[str, List[float]]] = {}
        for (disp, ctr), v in per.items():
            k = short_name(names[disp])
            byk.setdefault(k, {}).setdefault(ctr, []).append(v)
        for k, cs in byk.items():
            for ctr, vals in cs.items():
                table.setdefault(k, {})[ctr] = statistics.median(vals)
                calls[k] = max(calls.get(k, 0), len(vals))
    ctrs = sorted({c for cs in table.values() for c in cs})
    out = ["kernel | dispatches | " + " | ".join(ctrs), "---|---|" + "|".join("---" for _ in ctrs)]
    for k in sorted(table, key=lambda k: -calls[k]):
        out.append(f"{k} | {calls[k]} | " + " | ".join(f"{table[k].get(c, float('nan')):.4g}" for c in ctrs))
    return "\n".join(out)


def main(argv: List[str]) -> int:
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats_summary(argv[1]))
        return 0
    if len(argv) >= 2 and argv[0] == "counters":
        print(counters_summary(argv[1:]))
        return 0
    if len(argv) >= 5 and argv[0] == "traffic":
        t = traffic(argv[1], argv[2], argv[3], argv[5:] or None)
        with open(argv[4], "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
