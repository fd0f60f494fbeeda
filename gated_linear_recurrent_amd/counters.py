"""Summaries of rocprofv3 runs of bench.py for the notes kept under profiles/.

Kernel-time summary (from a `rocprofv3 --kernel-trace --stats` results database):

    python -m gated_linear_recurrent_amd.counters trace DB TITLE COMMAND > profiles/NAME.md

Counter record read by bench.py (from `rocprofv3 --pmc ... --output-format csv`
runs of `bench.py --copy-probe-mib MIB`: one run with FETCH_SIZE, one with
WRITE_SIZE, one with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE):

    python -m gated_linear_recurrent_amd.counters traffic --fetch DIR --write DIR --busy DIR \\
        --copy-mib MIB --command "..." --out profiles/traffic_counters.json

FETCH_SIZE and WRITE_SIZE are KiB per dispatch moved between the L2 and the
memory fabric. Each is scaled by the ratio of the known size of a plain
elementwise copy (torch.neg over MIB MiB of float32, reading and writing MIB
MiB) to what the same counter reads for that copy. MFMA busy is
SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE per XCD), with
GRBM_GUI_ACTIVE summed over the 8 XCDs.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel -> (name prefix in the trace, workload it was measured on, sources hashed)
KERNELS = {
    "prefill_output_kernel": ("liger::prefill_output_kernel<unsigned short, 128, 0, false>", "prefill_8b_b1_t8192_d128",
                              ["gated_linear_recurrent_amd/csrc/prefill.hip",
                               "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "prefill_output_kernel_vector_d128": ("liger::prefill_output_kernel<unsigned short, 128, 1, false>",
                                          "prefill_8b_b1_t32768_d128_outliers",
                                          ["gated_linear_recurrent_amd/csrc/prefill.hip",
                                           "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "prefill_output_kernel_vector_d64": ("liger::prefill_output_kernel<unsigned short, 64, 1, false>",
                                         "prefill_1b_b4_t2048_d64",
                                         ["gated_linear_recurrent_amd/csrc/prefill.hip",
                                          "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "segment_state_kernel": ("liger::segment_state_kernel<unsigned short, 128, 0>", "prefill_8b_b1_t8192_d128",
                             ["gated_linear_recurrent_amd/csrc/prefill.hip",
                              "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "decode_step_kernel": ("liger::decode_step_kernel<unsigned short, 128, 1, 4, false>", "decode_8b_n64_d128",
                           ["gated_linear_recurrent_amd/csrc/decode.hip",
                            "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "full_attn_kernel": ("liger::full_attn_kernel<128, 4>", "full_attn_8b_b1_t8192_d128",
                         ["gated_linear_recurrent_amd/csrc/full_attn.hip",
                          "gated_linear_recurrent_amd/csrc/device_common.h"]),
    "bwd_chunk_kernel": ("liger::bwd_chunk_kernel<128, 0>", "prefill_8b_b1_t8192_d128",
                         ["gated_linear_recurrent_amd/csrc/backward.hip",
                          "gated_linear_recurrent_amd/csrc/device_common.h"]),
}
N_SIMD = 1024
N_XCD = 8


def source_sha(files) -> str:
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    return re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "")).replace("void ", "")


def trace(db: str, title: str, command: str) -> str:
    cur = sqlite3.connect(db).cursor()
    rows = list(cur.execute("select name,total_calls,total_duration,average,percentage from top_kernels"))
    out = [f"# {title}\n", "Command (from the repository root, on the MI355X machine):\n", f"```\n{command}\n```\n",
           "| kernel | calls | total (us) | average (us) | % |", "|---|---|---|---|---|"]
    for n, c, t, a, p in rows:  # the view reports microseconds
        out.append(f"| `{_short(n)}` | {c} | {t:.1f} | {a:.2f} | {p:.1f} |")
    return "\n".join(out) + "\n"


def _counter_means(d: str) -> dict:
    """{kernel name: {counter: mean value per dispatch}} over every csv under d."""
    acc: dict = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = acc.setdefault(r["Kernel_Name"], {})
                k.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _find(means: dict, prefix: str) -> dict:
    for name, cs in means.items():
        if _short(name).startswith(prefix) or name.startswith(prefix) or prefix in name:
            return cs
    raise KeyError(prefix)


def traffic(fetch_dir: str, write_dir: str, busy_dir: str | None, copy_mib: int, command: str) -> dict:
    fetch, write = _counter_means(fetch_dir), _counter_means(write_dir)
    busy = _counter_means(busy_dir) if busy_dir else {}
    copy_kib = copy_mib * 1024.0
    f_copy = _find(fetch, "neg_kernel")["FETCH_SIZE"]
    w_copy = _find(write, "neg_kernel")["WRITE_SIZE"]
    sf, sw = copy_kib / f_copy, copy_kib / w_copy
    out = {"_calibration": {"copy_mib": copy_mib, "fetch_kib_read": f_copy, "write_kib_read": w_copy,
                            "fetch_scale": sf, "write_scale": sw, "command": command}}
    for kern, (prefix, workload, files) in KERNELS.items():
        try:
            fk = _find(fetch, prefix)["FETCH_SIZE"]
            wk = _find(write, prefix)["WRITE_SIZE"]
        except KeyError:
            continue
        rec = {"workload": workload, "source_sha256": source_sha(files),
               "fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
               "hbm_bytes_per_launch": (fk * sf + wk * sw) * 1024.0}
        try:
            b = _find(busy, prefix)
            rec["mfma_busy_frac"] = b["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * b["GRBM_GUI_ACTIVE"] / N_XCD)
        except KeyError:
            pass
        out[kern] = rec
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("title")
    t.add_argument("command")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--busy")
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--command", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace(a.db, a.title, a.command))
    else:
        rec = traffic(a.fetch, a.write, a.busy, a.copy_mib, a.command)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
