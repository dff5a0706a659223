"""Summaries of rocprofv3 output for the layer kernels (kernel times and HBM byte counters).

Used to turn the CSV files of

    rocprofv3 --kernel-trace --stats -f csv -d DIR -o layer -- python bench.py ...
    rocprofv3 --pmc FETCH_SIZE -f csv -d DIR -o layer -- python bench.py ... --copy-calibration
    rocprofv3 --pmc WRITE_SIZE -f csv -d DIR -o layer -- python bench.py ... --copy-calibration

into the short text summaries kept with the project, and to read them back.  The counter summary
records a hash of the batch-1 layer kernels' sources (common.hpp, predict.hip, select.hip,
ffn.hip): the benchmark reports the measured HBM traffic only while those are unchanged since the
counters were taken.

Counter scaling: FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by
the ratio of the known size of a plain device copy (the benchmark's --copy-calibration leg, a
1 GiB copy) to what the same counter reads for that copy.

    python -m contextual_sparsity_ffn_amd.profiling stats DIR/layer_kernel_stats.csv OUT.md "CMD" ["TITLE"]
    python -m contextual_sparsity_ffn_amd.profiling counters FETCH.csv WRITE.csv OUT.json OUT.md "CMD"
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30

# kernel-name prefix -> label used by the benchmark
LABELS = [("k_pred_down", "pred_down"), ("k_pred_up_select", "pred_up_select"),
          ("k_pred_up_loop", "pred_up"), ("k_pred_up", "pred_up"), ("k_select_topk", "select_topk"),
          ("k_select_threshold", "select_threshold"), ("k_gather_up", "gather_up"),
          ("k_gather_down", "gather_down"), ("k_reduce_partials", "reduce_partials"),
          ("k_ffn_fused", "ffn_fused"),
          ("k_pred_down_mfma", "pred_down_mfma"), ("k_pred_hidden", "pred_hidden"),
          ("k_pred_up_mfma_res", "pred_up_mfma"), ("k_pred_up_mfma", "pred_up_mfma"), ("k_union_list", "union_list"),
          ("k_union_up_valu", "union_up_valu"), ("k_union_down_valu", "union_down_valu"),
          ("k_union_up_lds", "union_up_mfma"), ("k_union_down_mfma", "union_down_mfma"),
          ("k_rms_norm", "rms_norm"), ("k_head_proj", "head_proj"), ("k_head_attn", "head_attn"),
          ("k_head_combine", "head_combine"), ("k_wide_hist", "select_hist"),
          ("k_wide_finish", "select_finish"),
          ("k_wide_zero", "select_zero")]


# the sources of the batch-1 layer kernels whose counters are kept (their code and launch shapes)
LAYER_SOURCES = ("common.hpp", "predict.hip", "select.hip", "ffn.hip")


def source_hash(names=LAYER_SOURCES) -> str:
    """SHA-256 over the named kernel sources in csrc/, in name order."""
    h = hashlib.sha256()
    for name in sorted(names):
        path = os.path.join(PKG, "csrc", name)
        h.update(name.encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def label_of(name: str):
    for prefix, label in LABELS:
        if re.search(r"\b" + prefix + r"\b", name):
            return label
    return None


def summarize_kernel_stats(stats_csv: str, out_md: str, command: str,
                           title: str = "contextual-sparsity layer kernels") -> None:
    rows = []
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            lab = label_of(r["Name"])
            if lab:
                rows.append((lab, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Name"]))
    rows.sort(key=lambda t: -t[1] * t[2])
    with open(out_md, "w") as out:
        out.write(f"# rocprofv3 kernel statistics: {title}\n\n")
        out.write(f"Command (repository root):\n\n    {command}\n\n")
        out.write(f"Kernel source sha256: `{source_hash()}`\n\n")
        out.write("| kernel | calls | avg us | min us | max us |\n|---|---:|---:|---:|---:|\n")
        for lab, calls, avg, mn, mx, _ in rows:
            out.write(f"| {lab} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} |\n")
        out.write("\nFull kernel names:\n\n")
        for lab, *_, name in rows:
            out.write(f"- {lab}: `{name}`\n")


def _per_dispatch(counter_csv: str, counter: str):
    out = []
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _copy_scale(disp) -> float:
    """Known bytes of the calibration copy over the counter's reading for it (KiB -> bytes)."""
    best = None
    for name, grid, kib in disp:
        # the runtime's device-to-device blit kernel; the largest one is the 1 GiB copy
        if "copyBuffer" in name and (best is None or kib > best):
            best = kib
    if not best:
        raise ValueError("no calibration copy dispatch found (run the benchmark with --copy-calibration)")
    return COPY_BYTES / (best * 1024.0)


def summarize_counters(fetch_csv: str, write_csv: str, out_json: str, out_md: str, command: str,
                       title: str = "layer kernels", sources=LAYER_SOURCES) -> dict:
    fetch, write = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    fs, ws = _copy_scale(fetch), _copy_scale(write)
    kern = {}
    for label in [l for _, l in LABELS]:
        fv = [kib for n, g, kib in fetch if label_of(n) == label]
        wv = [kib for n, g, kib in write if label_of(n) == label]
        if fv and wv:
            kern[label] = {"dispatches": len(fv),
                           "fetch_bytes": statistics.median(fv) * 1024.0 * fs,
                           "write_bytes": statistics.median(wv) * 1024.0 * ws}
    res = {"source_sha256": source_hash(sources), "sources": sorted(sources),
           "fetch_scale": fs, "write_scale": ws,
           "copy_bytes": COPY_BYTES, "command": command, "kernels": kern}
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
    with open(out_md, "w") as out:
        out.write(f"# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE), {title}\n\n")
        out.write(f"Command (repository root), once per counter:\n\n    {command}\n\n")
        out.write(f"Scale factors from the {COPY_BYTES >> 20} MiB calibration copy: FETCH_SIZE x{fs:.4f}, "
                  f"WRITE_SIZE x{ws:.4f} (counter KiB -> bytes: KiB * 1024 * factor).\n\n")
        out.write(f"Kernel source sha256 ({', '.join(res['sources'])}): `{res['source_sha256']}`\n\n")
        out.write("| kernel | dispatches | fetch MB (median) | write MB (median) |\n|---|---:|---:|---:|\n")
        for lab, v in kern.items():
            out.write(f"| {lab} | {v['dispatches']} | {v['fetch_bytes'] / 1e6:.3f} | {v['write_bytes'] / 1e6:.3f} |\n")
    return res


def load_counters(path: str):
    """The committed counter summary, or None if missing or taken from different kernel sources."""
    try:
        with open(path) as fh:
            res = json.load(fh)
    except (OSError, ValueError):
        return None
    return res if res.get("source_sha256") == source_hash() else None


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "stats":
        summarize_kernel_stats(sys.argv[2], sys.argv[3], sys.argv[4], *sys.argv[5:6])
    elif len(sys.argv) >= 2 and sys.argv[1] == "counters":
        extra = {}
        if len(sys.argv) >= 8:
            extra["title"] = sys.argv[7]
        if len(sys.argv) >= 9:
            extra["sources"] = tuple(sys.argv[8].split(","))
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], **extra)
    else:
        print(__doc__)
        sys.exit(2)
