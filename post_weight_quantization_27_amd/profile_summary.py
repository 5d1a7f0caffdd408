"""Summaries of rocprofv3 output for the pwq library calls.

Maps each GPU kernel of a run to the library call that launched it, and writes:

* ``stats``   : a Markdown table of the kernel-trace statistics (one row per kernel, with
  its call), plus per-call kernel time per step of the path (a step calls recon_mse twice,
  every other call once), to set beside the per-call durations the bench measures with HIP
  events;
* ``traffic`` : HBM bytes per call from two counter runs (``FETCH_SIZE``, then
  ``WRITE_SIZE``, KiB per dispatch), each scaled by what the same counter reads for a plain
  1 GiB device copy; stored as JSON with a hash of the kernel sources, so a reader can tell
  when the kernels have changed since the counters were taken.

Usage (the CSV files are rocprofv3's ``--output-format csv`` results)::

    python -m post_weight_quantization_27_amd.profile_summary stats STATS.csv \\
        --steps N --cmd "..." --out profiles/NAME.md
    python -m post_weight_quantization_27_amd.profile_summary traffic FETCH.csv WRITE.csv \\
        CFETCH.csv CWRITE.csv --steps N --workload W --layer L --cmd "..." --out profiles/traffic.json

N is the number of steps of the path the profiled run executed (bench.py prints it as
``path_steps_run``).  Per-kernel entries (the classes of the library's timing record: the
Hessian's contraction, the trailing updates, the column blocks) hold the summed bytes over
every dispatch of the run and the dispatch count, so bytes per launch need no step count.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))

# kernel-name fragments -> library call (first match wins; the bench's own H.zero_() fill
# is timed inside its hessian_accumulate events, so it is attributed there)
CALL_OF = [
    ("EpiHess", "hessian_accumulate"), ("hess_reduce", "hessian_accumulate"),
    ("mirror_upper", "hessian_accumulate"), ("transpose_bf16", "hessian_accumulate"),
    ("transpose_split", "hessian_accumulate"), ("FillFunctor", "hessian_accumulate"),
    ("damp_kernel", "hessian_damp"), ("act_order_kernel", "act_order_perm"), ("act_order_lds", "act_order_perm"),
    ("copy_upper", "chol_inverse_upper"), ("copy_perm", "chol_inverse_upper"), ("set_int", "chol_inverse_upper"),
    ("chol_diag", "chol_inverse_upper"), ("chol_update_diag", "chol_inverse_upper"),
    ("chol_split3", "chol_inverse_upper"),
    ("EpiStore", "chol_inverse_upper"), ("EpiSyrk", "chol_inverse_upper"), ("EpiPush", "chol_inverse_upper"),
    ("gptq_", "gptq_quantize_layer"), ("EpiSub", "gptq_quantize_layer"), ("inv_perm", "gptq_quantize_layer"),
    ("unpermute_codes", "gptq_quantize_layer"),
    ("rtn_kernel", "rtn_quantize"), ("rtn_group", "rtn_quantize"),
    ("dequant_kernel", "dequant"), ("dequant_vec", "dequant"), ("dequant_f16", "dequant"),
    ("mse_", "recon_mse"), ("EpiSq", "recon_mse"), ("set_double", "recon_mse"),
    ("SplitTriMap", "recon_mse"), ("EpiTrace", "recon_mse"),
    ("w4a16", "quantized_matmul"),
    ("chan_abs", "channel_abs_mean"), ("chan_mean", "channel_abs_mean"),
    ("awq_", "awq_search"), ("EpiDot", "awq_search"),
    ("tensor_max", "tensor_scales"), ("tensor_scale", "tensor_scales"),
]


# kernel-name fragments -> kernel class of the library's timing record (pwq_profile_read)
CLASS_OF = [("EpiHess", "xtx"), ("DlTiled6, DlTiled6, XcdRectMap, EpiSub", "update_split"),
            ("gptq_split3", "update_split_pieces"), ("EpiSub", "update"), ("gptq_block_kernel", "columns"),
            ("gptq_row_kernel", "columns")]


def class_of(name: str):
    # counter runs name kernels with their namespaces, kernel traces without
    name = name.replace("(anonymous namespace)::", "").replace("pwq::", "")
    for frag, cls in CLASS_OF:
        if frag in name:
            return cls
    return None


def call_of(name: str) -> str:
    for frag, call in CALL_OF:
        if frag in name:
            return call
    return "other"


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def source_hash() -> str:
    """sha256 over the kernel sources (csrc/*.hip, *.h) and the public header, with comments
    and blank space removed, so an edit of the prose alone keeps the counters valid."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) + glob.glob(os.path.join(HERE, "csrc", "*.h")))
    files.append(os.path.join(os.path.dirname(HERE), "include", "pwq.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def code_only(text: str) -> str:
    """C/HIP source text without its comments, runs of blank space made one space."""
    return " ".join(_COMMENT.sub(" ", text).split())


def short(name: str, n: int = 110) -> str:
    name = name.replace("pwq::(anonymous namespace)::", "").replace("pwq::", "")
    return name if len(name) <= n else name[: n - 3] + "..."


def stats(a) -> None:
    rows = list(csv.DictReader(open(a.stats_csv)))
    per_call = defaultdict(float)
    launches = defaultdict(int)
    lines = [f"# Kernel trace summary\n", f"Command: `{a.cmd}`\n",
             f"Kernel sources hash: `{source_hash()}`\n",
             "| kernel | call | launches | avg us | total us | % |", "|---|---|---|---|---|---|"]
    for r in rows:
        c = call_of(r["Name"])
        tot = float(r["TotalDurationNs"]) / 1e3
        per_call[c] += tot
        launches[c] += int(r["Calls"])
        lines.append(f"| `{short(r['Name'])}` | {c} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{tot:.1f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"Per library call, per step of the path ({a.steps} steps ran; kernel time summed):", "",
              "| call | kernel launches per step | kernel ms per step |", "|---|---|---|"]
    for c, t in sorted(per_call.items(), key=lambda kv: -kv[1]):
        lines.append(f"| {c} | {launches[c] / a.steps:.1f} | {t / a.steps / 1e3:.4f} |")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_sum(path: str) -> dict:
    """call -> summed counter value (KiB) over all dispatches."""
    out = defaultdict(float)
    for r in csv.DictReader(open(path)):
        out[call_of(r["Kernel_Name"])] += float(r["Counter_Value"])
    return out


def _class_sum(path: str):
    """kernel class -> (summed counter value, dispatches)."""
    val, cnt = defaultdict(float), defaultdict(int)
    for r in csv.DictReader(open(path)):
        c = class_of(r["Kernel_Name"])
        if c:
            val[c] += float(r["Counter_Value"])
            cnt[c] += 1
    return val, cnt


def _copy_factor(path: str, nbytes: int) -> float:
    """bytes per counter unit, from the 1 GiB copy dispatches of the calibration run."""
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy dispatch in {path}")
    return nbytes / (sum(vals) / len(vals))


def traffic(a) -> None:
    fetch, write = _counter_sum(a.fetch_csv), _counter_sum(a.write_csv)
    ff = _copy_factor(a.cfetch_csv, 1 << 30)
    fw = _copy_factor(a.cwrite_csv, 1 << 30)
    calls = {}
    for c in sorted(set(fetch) | set(write)):
        calls[c] = {"fetch_bytes": fetch.get(c, 0.0) * ff / a.steps, "write_bytes": write.get(c, 0.0) * fw / a.steps}
        calls[c]["hbm_bytes"] = calls[c]["fetch_bytes"] + calls[c]["write_bytes"]
    (kf, nf), (kw, nw) = _class_sum(a.fetch_csv), _class_sum(a.write_csv)
    kernels = {}
    for c in sorted(set(kf) | set(kw)):
        kernels[c] = {"fetch_bytes": kf.get(c, 0.0) * ff, "write_bytes": kw.get(c, 0.0) * fw,
                      "launches": nf.get(c, 0)}
        kernels[c]["hbm_bytes"] = kernels[c]["fetch_bytes"] + kernels[c]["write_bytes"]
        if nf.get(c, 0) != nw.get(c, 0):
            raise SystemExit(f"{c}: {nf.get(c, 0)} dispatches in the FETCH run, {nw.get(c, 0)} in the WRITE run")
    data = {}
    if os.path.exists(a.out):
        data = json.load(open(a.out))
    data[f"{a.workload}/{a.layer}"] = {
        "command": a.cmd, "source_hash": source_hash(), "steps_run": a.steps,
        "fetch_bytes_per_counter_unit": ff, "write_bytes_per_counter_unit": fw, "per_call": calls,
        "per_kernel": kernels}
    with open(a.out, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--steps", type=int, required=True, help="steps of the path the run executed")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch_csv", "write_csv", "cfetch_csv", "cwrite_csv"):
        t.add_argument(k)
    t.add_argument("--steps", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--layer", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args()
    stats(a) if a.mode == "stats" else traffic(a)


if __name__ == "__main__":
    main()
