"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m discrete_text_diffusion_denoise_amd.profiling trace DIR
        per-kernel table (calls, total, average, min, max) from the
        --kernel-trace CSV in DIR (markdown)

    python -m discrete_text_diffusion_denoise_amd.profiling counters KERNEL DIR [DIR ...]
        every PMC counter found in the --pmc runs in DIR..., averaged per
        dispatch of KERNEL (one line per counter)

    python -m discrete_text_diffusion_denoise_amd.profiling traffic FETCH_DIR WRITE_DIR KERNEL
        HBM traffic of KERNEL per dispatch from a FETCH_SIZE run and a
        WRITE_SIZE run, each scaled by what the same counter reads for the
        1 GiB device-to-device copies that `bench.py --copy-probe` issues
        (the counters do not report bytes one to one on this part)

Kernel names are matched by substring of the demangled name.
"""
from __future__ import annotations

import csv
import glob
import os
import re
import sys

COPY_BYTES = 1 << 30          # one copy of bench.py --copy-probe
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def short_name(k: str) -> str:
    m = re.search(r"namespace\)::([A-Za-z0-9_]+)(<[^(]*)?", k)
    if m:
        return m.group(1) + (m.group(2) or "")
    return k.split("(")[0][:80]


def kernel_table(d: str):
    rows = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    agg: dict[str, list[float]] = {}
    for r in rows:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault(short_name(r["Kernel_Name"]), []).append(us)
    total = sum(sum(v) for v in agg.values())
    out = []
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append((k, len(v), sum(v), sum(v) / len(v), min(v), max(v), 100.0 * sum(v) / total))
    return out


def counter_per_dispatch(d: str, counter: str, kernel: str):
    """Average value of `counter` over dispatches whose name contains
    `kernel`, and over the large copies (the calibration)."""
    rows = [r for r in csv.DictReader(open(_find(d, "counter_collection.csv")))
            if r["Counter_Name"] == counter]
    kv = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
    cp = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]]
    if not kv:
        raise ValueError(f"no {counter} dispatches of {kernel}")
    big = max(cp) if cp else 0.0
    cp = [c for c in cp if c > 0.5 * big]
    return sum(kv) / len(kv), len(kv), (sum(cp) / len(cp) if cp else None), len(cp)


def counters(kernel: str, dirs) -> dict:
    """{counter: (average per dispatch of `kernel`, dispatches)} over every
    counter recorded in the --pmc runs under `dirs`."""
    acc: dict[str, list[float]] = {}
    for d in dirs:
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            if kernel in r["Kernel_Name"]:
                acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in sorted(acc.items())}


def traffic(fetch_dir: str, write_dir: str, kernel: str) -> dict:
    f, nf, fc, nfc = counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    w, nw, wc, nwc = counter_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    # a D2D copy of COPY_BYTES reads and writes COPY_BYTES each
    rf = COPY_BYTES / (fc * 1024.0) if fc else None
    rw = COPY_BYTES / (wc * 1024.0) if wc else None
    out = {"kernel": kernel, "fetch_kib": f, "write_kib": w, "dispatches": [nf, nw],
           "copy_fetch_kib": fc, "copy_write_kib": wc, "copy_dispatches": [nfc, nwc],
           "fetch_scale": rf, "write_scale": rw}
    if rf and rw:
        out["read_bytes"] = f * 1024.0 * rf
        out["write_bytes"] = w * 1024.0 * rw
        out["traffic_bytes"] = out["read_bytes"] + out["write_bytes"]
    return out


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print("| total ms | % | calls | avg us | min us | max us | kernel |")
        print("|---:|---:|---:|---:|---:|---:|---|")
        for k, n, tot, avg, mn, mx, pct in kernel_table(argv[1]):
            print(f"| {tot / 1e3:.3f} | {pct:.1f} | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | `{k}` |")
        return 0
    if len(argv) >= 3 and argv[0] == "counters":
        for k, (v, n) in counters(argv[1], argv[2:]).items():
            print(f"{k}: {v:.6g}  ({n} dispatches)")
        return 0
    if len(argv) >= 4 and argv[0] == "traffic":
        t = traffic(argv[1], argv[2], argv[3])
        for k, v in t.items():
            print(f"{k}: {v}")
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
