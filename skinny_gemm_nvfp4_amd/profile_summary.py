"""Summaries of rocprofv3 output for the NVFP4 GEMM kernels (text for profiles/, JSON for bench).

Inputs are the CSV files rocprofv3 writes with ``-f csv``:
  * kernel trace (``--kernel-trace``): one row per dispatch with start/end timestamps in ns;
  * counter collection (``--pmc``): one or more rows per dispatch and counter.

GEMM dispatches are the kernels of the ``nvfp4::`` namespace other than the pack kernels. They
are matched in launch order with the labels ``bench.py --launch-log`` wrote, so every duration
and counter is attributed to a named GEMM of a named workload. A call of two dispatches (the
greedy-token call: GEMM then ``argmax_finalize_kernel``; a fused call above the dot-product rows:
``rmsnorm_rows_kernel`` then the GEMM) counts as one: the duration spans both, counters are
summed.

HBM traffic: FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch but, on this part, do not
necessarily count every memory channel; each is therefore scaled by bytes / counter of the
calibration copy bench.py runs first (the first ``__amd_rocclr_copyBuffer`` dispatch of about
that size, a plain device-to-device copy of ``--calibration-bytes``).

MFMA busy (``mfma``): SQ_VALU_MFMA_BUSY_CYCLES counts the matrix-core busy cycles of every SIMD
(16 per v_mfma_f32_16x16x32_bf16); GRBM_GUI_ACTIVE counts the active cycles of the dispatch,
summed over the XCDs. Busy fraction = MFMA busy / (SIMDs x GRBM_GUI_ACTIVE / XCDs).

Usage:
  python -m skinny_gemm_nvfp4_amd.profile_summary trace --trace T.csv --labels L.txt
  python -m skinny_gemm_nvfp4_amd.profile_summary mfma --counters C.csv --labels L.txt
  python -m skinny_gemm_nvfp4_amd.profile_summary traffic --fetch F.csv --write W.csv \
      --labels L.txt [--calibration-bytes B] [--json profiles/traffic.json]
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys
from collections import OrderedDict

PACK_KERNELS = ("pack_clear_kernel", "pack_amax_kernel", "pack_scale_kernel",
                "pack_quant_kernel")
# Dispatches that finish a GEMM call started by the dispatch before them: the greedy-token
# finalize of nvfp4_gemm_argmax.
FOLLOW_KERNELS = ("argmax_finalize_kernel",)
# Dispatches that open a GEMM call whose GEMM dispatch comes next: the row-wise RMSNorm of a
# fused call that does not normalise inside the dot-product kernel.
LEAD_KERNELS = ("rmsnorm_rows_kernel",)
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def is_gemm(name: str) -> bool:
    return "nvfp4::" in name and not any(p in name for p in PACK_KERNELS)


def short_name(name: str) -> str:
    name = name.replace("void ", "").replace("nvfp4::", "")
    return name.split("(")[0]


def read_labels(path: str):
    with open(path) as f:
        return [line.strip() for line in f if line.strip()]


def read_trace(path: str):
    """Dispatches of a kernel trace in start order: dicts with name, ns, grid, lds, regs."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({
                "id": int(r["Dispatch_Id"]),
                "name": r["Kernel_Name"],
                "start": int(r["Start_Timestamp"]),
                "end": int(r["End_Timestamp"]),
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                "grid": (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"])),
                "wg": int(r["Workgroup_Size_X"]),
                "lds": int(r["LDS_Block_Size"]),
                "vgpr": int(r["VGPR_Count"]), "agpr": int(r["Accum_VGPR_Count"]),
                "scratch": int(r["Scratch_Size"]),
            })
    rows.sort(key=lambda d: (d["start"], d["id"]))
    return rows


def read_counters(path: str):
    """Dispatches of a counter collection in dispatch order: dicts with name and counter sums."""
    per = OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                       "grid": int(r["Grid_Size"])})
            c = r["Counter_Name"]
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def is_follow(name: str) -> bool:
    return any(f"nvfp4::{k}" in name for k in FOLLOW_KERNELS)


def is_lead(name: str) -> bool:
    return any(f"nvfp4::{k}" in name for k in LEAD_KERNELS)


def _merge(into, d):
    """Adds dispatch d to the call `into`: the span covers both, counters are summed."""
    if "start" in d and "start" in into:
        into["start"] = min(into["start"], d["start"])
        into["end"] = max(into["end"], d["end"])
        into["ns"] = into["end"] - into["start"]
    for k, v in d.items():
        if k.isupper() and isinstance(v, float):
            into[k] = into.get(k, 0.0) + v


def fold_reductions(gemms):
    """Folds each follow-on dispatch (argmax finalize) into the GEMM dispatch before it, and each
    lead dispatch (RMSNorm) into the GEMM dispatch after it."""
    out = []
    lead = None
    for d in gemms:
        if is_lead(d["name"]):
            lead = d
            continue
        if lead is not None and not is_follow(d["name"]):
            _merge(d, lead)
            d["fused"] = True
            lead = None
        if is_follow(d["name"]):
            if not out:
                raise ValueError("a follow-on dispatch with no GEMM dispatch before it")
            prev = out[-1]
            if "end" in d and "start" in prev:   # kernel trace: span of both dispatches
                prev["end"] = d["end"]
                prev["ns"] = prev["end"] - prev["start"]
            for k, v in d.items():               # counter collection: sums
                if k.isupper() and isinstance(v, float):
                    prev[k] = prev.get(k, 0.0) + v
            if "argmax" in d["name"]:
                prev["argmax"] = True
            continue
        out.append(d)
    if lead is not None:
        raise ValueError("a lead dispatch with no GEMM dispatch after it")
    return out


def attach_labels(dispatches, labels):
    """Pairs the GEMM dispatches with the launch log. Raises if the counts differ."""
    gemms = fold_reductions([d for d in dispatches if is_gemm(d["name"])])
    if len(gemms) != len(labels):
        raise ValueError(f"{len(gemms)} GEMM dispatches in the profile but {len(labels)} "
                         "labels in the launch log")
    for d, lab in zip(gemms, labels):
        d["label"] = lab
    return gemms


def group(gemms):
    out = OrderedDict()
    for d in gemms:
        out.setdefault(d["label"], []).append(d)
    return out


def trace_summary(trace_csv: str, labels_path: str) -> str:
    gemms = attach_labels(read_trace(trace_csv), read_labels(labels_path))
    lines = [f"{'GEMM':44s} {'kernel':56s} {'n':>4s} {'mean_us':>8s} {'med_us':>8s} "
             f"{'min_us':>8s}  grid        wg   lds    vgpr agpr scratch"]
    for lab, ds in group(gemms).items():
        us = [d["ns"] / 1e3 for d in ds]
        d0 = ds[0]
        kname = (short_name(d0["name"]) + (" +argmax" if d0.get("argmax") else "") +
                 (" +norm" if d0.get("fused") else ""))
        lines.append(
            f"{lab:44s} {kname[:56]:56s} {len(us):4d} "
            f"{statistics.fmean(us):8.2f} {statistics.median(us):8.2f} {min(us):8.2f}  "
            f"{d0['grid'][0]:>5d}x{d0['grid'][1]:<4d} {d0['wg']:5d} {d0['lds']:6d} "
            f"{d0['vgpr']:4d} {d0['agpr']:4d} {d0['scratch']:6d}")
    return "\n".join(lines)


MI355X_SIMDS = 256 * 4    # 256 compute units of 4 SIMDs
MI355X_XCDS = 8


def mfma_summary(counters_csv: str, labels_path: str) -> str:
    gemms = attach_labels(read_counters(counters_csv), read_labels(labels_path))
    lines = [f"{'GEMM':48s} {'n':>4s} {'MFMA instr':>11s} {'busy cycles':>12s} "
             f"{'active cyc':>11s} {'busy %':>7s}"]
    for lab, ds in group(gemms).items():
        med = {k: statistics.median(d.get(k, 0.0) for d in ds)
               for k in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
        active = med["GRBM_GUI_ACTIVE"] / MI355X_XCDS
        frac = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (MI355X_SIMDS * active) if active else 0.0
        lines.append(f"{lab:48s} {len(ds):4d} {med['SQ_INSTS_MFMA']:11.4g} "
                     f"{med['SQ_VALU_MFMA_BUSY_CYCLES']:12.4g} {active:11.4g} {100 * frac:7.1f}")
    return "\n".join(lines)


def calibration(dispatches, counter: str, nbytes: int) -> float:
    """bytes / counter bytes of the calibration copy: the FIRST copy dispatch whose counter is at
    least 1/64 of `nbytes` (bench.py copies before anything else; later device-to-device copies,
    such as cloned weight copies, may be larger and must not be taken for it; a counter may see
    only a fraction of the channels)."""
    copies = [d for d in dispatches if d["name"].startswith(COPY_KERNEL) and counter in d]
    big = [d for d in copies if d[counter] * 1024.0 >= nbytes / 64]
    if not big:
        raise ValueError(f"no {COPY_KERNEL} dispatch of the calibration size with {counter}")
    return nbytes / (big[0][counter] * 1024.0)


def traffic_summary(fetch_csv: str, write_csv: str, labels_path: str, nbytes: int):
    labels = read_labels(labels_path)
    fetch = read_counters(fetch_csv)
    write = read_counters(write_csv)
    kf = calibration(fetch, "FETCH_SIZE", nbytes)
    kw = calibration(write, "WRITE_SIZE", nbytes)
    gf = group(attach_labels(fetch, labels))
    gw = group(attach_labels(write, labels))
    rows = OrderedDict()
    for lab in gf:
        f_b = statistics.median(d["FETCH_SIZE"] for d in gf[lab]) * 1024.0 * kf
        w_b = statistics.median(d["WRITE_SIZE"] for d in gw[lab]) * 1024.0 * kw
        rows[lab] = {"kernel": short_name(gf[lab][0]["name"]), "n": len(gf[lab]),
                     "fetch_bytes": round(f_b), "write_bytes": round(w_b),
                     "bytes_per_launch": round(f_b + w_b)}
    return kf, kw, rows


def _algorithmic_bytes(label: str):
    from .roofline import compulsory_bytes
    try:
        dims = dict(part.split("=") for part in label.split()[1:])
        return compulsory_bytes(int(dims["M"]), int(dims["N"]), int(dims["K"]))
    except (KeyError, ValueError):
        return None


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--trace", required=True)
    t.add_argument("--labels", required=True)
    w = sub.add_parser("traffic")
    w.add_argument("--fetch", required=True)
    w.add_argument("--write", required=True)
    w.add_argument("--labels", required=True)
    w.add_argument("--calibration-bytes", type=int, default=256 << 20)
    w.add_argument("--json", default=None, help="also merge bytes per launch into this file")
    m = sub.add_parser("mfma")
    m.add_argument("--counters", required=True)
    m.add_argument("--labels", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        print(trace_summary(args.trace, args.labels))
        return 0
    if args.cmd == "mfma":
        print(mfma_summary(args.counters, args.labels))
        return 0
    kf, kw, rows = traffic_summary(args.fetch, args.write, args.labels, args.calibration_bytes)
    print(f"calibration: FETCH_SIZE x {kf:.4f}, WRITE_SIZE x {kw:.4f} "
          f"(bytes of the {args.calibration_bytes}-byte copy / counter bytes)")
    print(f"{'GEMM':44s} {'n':>3s} {'fetch_MB':>9s} {'write_MB':>9s} {'total_MB':>9s} "
          f"{'algo_MB':>9s} {'total/algo':>10s}")
    for lab, r in rows.items():
        algo = _algorithmic_bytes(lab)
        ratio = f"{r['bytes_per_launch'] / algo:10.3f}" if algo else f"{'-':>10s}"
        print(f"{lab:44s} {r['n']:3d} {r['fetch_bytes'] / 1e6:9.3f} "
              f"{r['write_bytes'] / 1e6:9.3f} {r['bytes_per_launch'] / 1e6:9.3f} "
              f"{(algo or 0) / 1e6:9.3f} {ratio}")
    if args.json:
        data = {}
        if os.path.exists(args.json):
            with open(args.json) as f:
                data = json.load(f)
        h = source_hash()
        for lab, r in rows.items():
            data[lab] = dict(r, source_hash=h)
        with open(args.json, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
