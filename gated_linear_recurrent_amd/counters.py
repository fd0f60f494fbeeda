"""Summaries of rocprofv3 runs of bench.py for the notes kept under profiles/.

Kernel-time summary (from a `rocprofv3 --kernel-trace --stats` results database):

    python -m gated_linear_recurrent_amd.counters trace DB TITLE COMMAND > profiles/NAME.md

Counter record read by bench.py (from `rocprofv3 --pmc ... --output-format csv`
runs of `bench.py --copy-probe-mib MIB`: one run with FETCH_SIZE, one with
WRITE_SIZE, one with the SQ busy counters and GRBM_GUI_ACTIVE, optionally one
with the L2-to-fabric read request counters):

    python -m gated_linear_recurrent_amd.counters traffic --fetch DIR --write DIR --busy DIR \\
        [--tcc DIR] --copy-mib MIB --command "..." --out profiles/traffic_counters.json

FETCH_SIZE and WRITE_SIZE are KiB per dispatch moved between the L2 and the
memory fabric. Each is scaled by the ratio of the known size of a plain
elementwise copy (torch.neg over MIB MiB of float32, reading and writing MIB
MiB) to what the same counter reads for that copy. The busy fractions follow
the derived metrics rocprofv3 lists for gfx950 (GRBM_GUI_ACTIVE per XCD being
the csv value, summed over the 8 XCDs, divided by 8):
  MFMA busy        SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE)   (MfmaUtil)
  VALU busy        SQ_ACTIVE_INST_VALU / (256 CUs x GRBM_GUI_ACTIVE)           (VALUBusy)
  LDS conflict     SQ_LDS_BANK_CONFLICT / (256 CUs x GRBM_GUI_ACTIVE)          (LDSBankConflict)
  conflicts/access SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)
The read pass gives the mean time an L2 miss is outstanding, in cycles:
TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum (requests in flight summed per
cycle over requests, Little's law). The decode kernel's dispatches are also
split by the dispatch that ran just before each one: the cache-evicting read
(a reduction), the evicting write (a fill), or another decode step.

Summary table of a record:

    python -m gated_linear_recurrent_amd.counters summary profiles/traffic_counters.json
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
    "segment_state_scalar_kernel": ("liger::segment_state_scalar_kernel<unsigned short, 128>", "prefill_8b_b1_t8192_d128",
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
N_CU = 256
N_XCD = 8
# name fragments of the kernels that run right before a decode step in each regime
DECODE_REGIMES = {"after_read_eviction": "reduce_kernel", "after_write_eviction": "FillFunctor",
                  "back_to_back": "decode_step_kernel"}


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


def _dispatches(d: str) -> list:
    """[(dispatch id, kernel name, {counter: value})] over every csv under d, in dispatch order."""
    by_id: dict = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (f, int(r["Dispatch_Id"]))
                name, cs = by_id.setdefault(key, (r["Kernel_Name"], {}))
                cs[r["Counter_Name"]] = float(r["Counter_Value"])
    return [(i, n, cs) for (_, i), (n, cs) in sorted(by_id.items())]


def _counter_means(d: str, after: str | None = None) -> dict:
    """{kernel name: {counter: mean value per dispatch}} over every csv under d;
    with `after`, only dispatches whose preceding dispatch's name contains it."""
    acc: dict = {}
    prev = None
    for _, name, cs in _dispatches(d):
        if after is None or (prev is not None and after in prev):
            k = acc.setdefault(name, {})
            for c, v in cs.items():
                k.setdefault(c, []).append(v)
        prev = name
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def busy_fracs(b: dict) -> dict:
    """Derived busy fractions of one kernel's SQ pass (see the module docstring)."""
    out = {}
    gui = b.get("GRBM_GUI_ACTIVE")
    if gui:
        per_xcd = gui / N_XCD
        if "SQ_VALU_MFMA_BUSY_CYCLES" in b:
            out["mfma_busy_frac"] = b["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * per_xcd)
        if "SQ_ACTIVE_INST_VALU" in b:
            out["valu_busy_frac"] = b["SQ_ACTIVE_INST_VALU"] / (N_CU * per_xcd)
        if "SQ_LDS_BANK_CONFLICT" in b:
            out["lds_bank_conflict_frac"] = b["SQ_LDS_BANK_CONFLICT"] / (N_CU * per_xcd)
    act, conf = b.get("SQ_LDS_IDX_ACTIVE"), b.get("SQ_LDS_BANK_CONFLICT")
    if act and conf is not None and act > conf:
        out["lds_conflicts_per_access"] = conf / (act - conf)
    return out


def read_latency(t: dict) -> dict:
    """Mean cycles an L2 read miss is outstanding, and the read requests per dispatch."""
    out = {}
    if t.get("TCC_EA0_RDREQ_sum"):
        out["read_requests"] = t["TCC_EA0_RDREQ_sum"]
        if "TCC_EA0_RDREQ_LEVEL_sum" in t:
            out["read_latency_cycles"] = t["TCC_EA0_RDREQ_LEVEL_sum"] / t["TCC_EA0_RDREQ_sum"]
        if "TCC_EA0_RDREQ_DRAM_sum" in t:
            out["dram_read_requests"] = t["TCC_EA0_RDREQ_DRAM_sum"]
    return out


def _find(means: dict, prefix: str) -> dict:
    for name, cs in means.items():
        if _short(name).startswith(prefix) or name.startswith(prefix) or prefix in name:
            return cs
    raise KeyError(prefix)


def traffic(fetch_dir: str, write_dir: str, busy_dir: str | None, copy_mib: int, command: str,
            tcc_dir: str | None = None) -> dict:
    fetch, write = _counter_means(fetch_dir), _counter_means(write_dir)
    busy = _counter_means(busy_dir) if busy_dir else {}
    tcc = _counter_means(tcc_dir) if tcc_dir else {}
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
            rec.update(busy_fracs(b))
            rec["sq"] = b
        except KeyError:
            pass
        try:
            rec.update(read_latency(_find(tcc, prefix)))
        except KeyError:
            pass
        if kern == "decode_step_kernel":
            rec["regimes"] = {}
            for regime, before in DECODE_REGIMES.items():
                r = {}
                try:
                    fk = _find(_counter_means(fetch_dir, before), prefix)["FETCH_SIZE"]
                    wk = _find(_counter_means(write_dir, before), prefix)["WRITE_SIZE"]
                    r["hbm_bytes_per_launch"] = (fk * sf + wk * sw) * 1024.0
                except KeyError:
                    pass
                for d, fn in ((busy_dir, busy_fracs), (tcc_dir, read_latency)):
                    if d:
                        try:
                            r.update(fn(_find(_counter_means(d, before), prefix)))
                        except KeyError:
                            pass
                rec["regimes"][regime] = r
        out[kern] = rec
    return out


def summary(rec: dict) -> str:
    """Markdown table of a traffic record."""
    cal = rec["_calibration"]
    lines = [f"Calibration: a plain elementwise copy of {cal['copy_mib']} MiB reads FETCH_SIZE = "
             f"{cal['fetch_kib_read']:,.0f} KiB and WRITE_SIZE = {cal['write_kib_read']:,.0f} KiB per dispatch, "
             f"so FETCH_SIZE is scaled by {cal['fetch_scale']:.3f} and WRITE_SIZE by {cal['write_scale']:.3f}.\n",
             "| kernel (workload) | HBM bytes/launch | MFMA busy | VALU busy | LDS bank-conflict stall | "
             "conflicts/access | L2 read miss latency (cycles) |",
             "|---|---|---|---|---|---|---|"]

    def pct(x):
        return "" if x is None else f"{100 * x:.1f}%"

    def row(name, r):
        hb = r.get("hbm_bytes_per_launch")
        lat = r.get("read_latency_cycles")
        cpa = r.get("lds_conflicts_per_access")
        return (f"| {name} | {'' if hb is None else f'{hb / 1e6:.1f} MB'} | {pct(r.get('mfma_busy_frac'))} | "
                f"{pct(r.get('valu_busy_frac'))} | {pct(r.get('lds_bank_conflict_frac'))} | "
                f"{'' if cpa is None else f'{cpa:.2f}'} | {'' if lat is None else f'{lat:.0f}'} |")

    for kern, r in rec.items():
        if kern.startswith("_"):
            continue
        lines.append(row(f"`{kern}` ({r['workload']})", r))
        for regime, rr in r.get("regimes", {}).items():
            lines.append(row(f"&nbsp;&nbsp;{kern}, {regime.replace('_', ' ')}", rr))
    return "\n".join(lines) + "\n"


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
    c.add_argument("--tcc")
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--command", default="")
    c.add_argument("--out", required=True)
    m = sub.add_parser("summary")
    m.add_argument("record")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace(a.db, a.title, a.command))
    elif a.cmd == "summary":
        with open(a.record) as f:
            sys.stdout.write(summary(json.load(f)))
    else:
        rec = traffic(a.fetch, a.write, a.busy, a.copy_mib, a.command, a.tcc)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
