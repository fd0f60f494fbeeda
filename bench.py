#!/usr/bin/env python3
"""Liger Attention throughput on one MI355X.

A step is one prefill of the Llama-3-8B-shaped workload
(B=1, T=8192, H_q=32, H_kv=8, d=128, bf16, scalar gate, window 64,
alpha 0.5) with its inputs already resident in device memory. The JSON
line reports prefill tokens/s as `value`, the roofline of the dominant kernel
(the fused output kernel, timed with HIP events on the stream it runs on),
the float64 CPU oracle on the host as a reported baseline, and the decode
workload (64 sequences, Llama-3-8B heads, one token per step) as extra keys.

    python bench.py [--steps K] [--warmup W] [--decode-steps N]

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PREFILL_WORKLOAD = "prefill_8b_b1_t8192_d128"
DECODE_WORKLOAD = "decode_8b_n64_d128"
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    "prefill_output_kernel": ["gated_linear_recurrent_amd/csrc/prefill.hip",
                              "gated_linear_recurrent_amd/csrc/device_common.h"],
    "decode_step_kernel": ["gated_linear_recurrent_amd/csrc/decode.hip",
                           "gated_linear_recurrent_amd/csrc/device_common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def prefill_algorithmic(cfg: dict) -> tuple[float, float]:
    """One read of q, k, v, one write of o and S_T; flops of the method itself.

    Per (batch, query head, token) with chunk C = 64 and window w:
      window 4 w d + intra-chunk 2 d (C + 1) + state->chunk 2 d^2 + chunk->state 2 d^2 / n_rep.
    """
    B, T, H_q, H_kv, d, w = cfg["B"], cfg["T"], cfg["H_q"], cfg["H_kv"], cfg["d"], cfg["window"]
    esz = 2 if cfg["dtype"] == "bf16" else 4
    n_rep = H_q // H_kv
    byts = B * T * (2 * H_q + 2 * H_kv) * d * esz + B * H_kv * d * d * 4
    flops = B * T * H_q * (4 * w * d + 2 * d * (CHUNK + 1) + 2 * d * d + 2 * d * d / n_rep)
    return float(byts), float(flops)


def decode_algorithmic(cfg: dict) -> float:
    """Bytes per step: state read + write, ring read of window-1 slots and write
    of one slot (k and v), q/k/v in, o out."""
    N, H_q, H_kv, d, w = cfg["N"], cfg["H_q"], cfg["H_kv"], cfg["d"], cfg["window"]
    esz = 2
    per_seq = (H_kv * 2 * d * d * 4 + H_kv * (w - 1) * d * esz * 2 + H_kv * d * esz * 2
               + 2 * H_q * d * esz + 2 * H_kv * d * esz)
    return float(N * per_seq)


def cpu_baseline(cfg: dict, x: dict, tokens: int) -> dict:
    """The float64 oracle as it stands, on the host, BLAS limited to one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    gate = 0 if cfg["gate"] == "scalar" else 1
    q, k, v = (x[n][:, :tokens] for n in ("q", "k", "v"))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, gate, cfg["window"], cfg["alpha"])
        dt = time.perf_counter() - t0
    return {"value": cfg["B"] * tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{PREFILL_WORKLOAD}: first {tokens} of {cfg['T']} tokens (all heads), float64 "
                      f"token loop, BLAS limited to 1 thread; {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-tokens", type=int, default=8192)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Liger Attention layer here is built and "
              "measured on a single MI355X; multi-GPU runs are not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gated_linear_recurrent_amd as gla
    from synth import CONFIGS, config_prefill_inputs, decode_initial, decode_step_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS[PREFILL_WORKLOAD]
    gate = gla.LIGER_GATE_SCALAR_MEAN if cfg["gate"] == "scalar" else gla.LIGER_GATE_VECTOR_AVGPOOL4
    log(f"[bench] generating {PREFILL_WORKLOAD}")
    x = config_prefill_inputs(PREFILL_WORKLOAD)
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous() for n in ("q", "k", "v"))
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    o = torch.empty_like(q)
    S_T = torch.empty((B, H_kv, d, d), dtype=torch.float32, device=dev)
    ws_bytes = gla.liger_attn_prefill_workspace_size(B, T, H_q, H_kv, d, gla.LIGER_BF16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def prefill(mask):
        gla.liger_attn_prefill(q, k, v, gate, cfg["window"], cfg["alpha"], o=o, S_T=S_T, workspace=ws,
                               stage_mask=mask)

    log(f"[bench] prefill warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill(7)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"[bench] prefill timed {args.steps}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        prefill(gla.LIGER_STAGE_SEGMENT_STATES | gla.LIGER_STAGE_CARRY_SCAN)
        e[1].record()
        prefill(gla.LIGER_STAGE_OUTPUT)
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    carry_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    out_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    byts, flops = prefill_algorithmic(cfg)
    achieved = byts / (out_ms * 1e-3) / 1e9
    traffic = measured_traffic("prefill_output_kernel", PREFILL_WORKLOAD)
    result = {
        "metric": "Liger Attention prefill tokens/s/GPU at 8B shapes; decode steps/s; % roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL_WORKLOAD, "B": B, "T": T, "H_q": H_q, "H_kv": H_kv, "d": d,
                   "gate": cfg["gate"], "window": cfg["window"], "alpha": cfg["alpha"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "prefill_output_kernel", "kernel_ms": out_ms,
                     "algorithmic_bytes": byts, "algorithmic_flops": flops,
                     "mfma_frac_algorithmic": flops / (out_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)},
        "prefill_breakdown_ms": {"segment_states_and_carry_scan": carry_ms, "output": out_ms,
                                 "events_total": carry_ms + out_ms},
        "prefill_op_roofline_frac": byts / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    log(f"[bench] prefill {ms_per_step * 1e3:.1f} us/step; output kernel {out_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s); carries {carry_ms * 1e3:.1f} us")

    if not args.no_decode:
        dcfg = CONFIGS[DECODE_WORKLOAD]
        dgate = gla.LIGER_GATE_SCALAR_MEAN if dcfg["gate"] == "scalar" else gla.LIGER_GATE_VECTOR_AVGPOOL4
        N, Hq, Hkv, dd, w = dcfg["N"], dcfg["H_q"], dcfg["H_kv"], dcfg["d"], dcfg["window"]
        nsteps = args.decode_steps
        log(f"[bench] generating {DECODE_WORKLOAD} ({nsteps} steps)")
        init = decode_initial(**dcfg)
        S = torch.from_numpy(init["S"]).to(dev)
        ring = gla.KVRing(torch.from_numpy(init["ring_k"]).to(dev).to(torch.bfloat16),
                          torch.from_numpy(init["ring_v"]).to(dev).to(torch.bfloat16),
                          torch.from_numpy(init["pos"]).to(dev), torch.zeros(N, dtype=torch.int32, device=dev), w)
        steps_in = []
        for s in range(nsteps):
            xs = decode_step_inputs(step=s, **dcfg)
            steps_in.append(tuple(torch.from_numpy(xs[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v")))
        do = torch.empty((N, Hq, dd), dtype=torch.bfloat16, device=dev)
        dwarm = min(16, nsteps)
        for s in range(dwarm):
            gla.liger_attn_decode_step(*steps_in[s], S, ring, dgate, dcfg["alpha"], o=do)
        torch.cuda.synchronize()
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
        t0 = time.perf_counter()
        for s in range(nsteps):
            dev_ev[s][0].record()
            gla.liger_attn_decode_step(*steps_in[s], S, ring, dgate, dcfg["alpha"], o=do)
            dev_ev[s][1].record()
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        k_ms = float(np.mean([a.elapsed_time(b) for a, b in dev_ev]))
        dbytes = decode_algorithmic(dcfg)
        dach = dbytes / (k_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": DECODE_WORKLOAD, "steps": nsteps, "warmup": dwarm,
            "steps_per_s": nsteps / dwall, "us_per_step_wall": dwall * 1e6 / nsteps,
            "kernel_us": k_ms * 1e3, "steps_per_s_kernel": 1e3 / k_ms,
            "tokens_per_s_kernel": N * 1e3 / k_ms,
            "roofline": {"bound": "hbm", "achieved": dach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": dach / PEAK_HBM_GBS,
                         "traffic": measured_traffic("decode_step_kernel", DECODE_WORKLOAD),
                         "kernel": "decode_step_kernel", "algorithmic_bytes": dbytes,
                         "note": "state + ring working set (48 MiB) fits the 256 MB last-level cache"},
        }
        log(f"[bench] decode kernel {k_ms * 1e3:.1f} us/step ({dach:.0f} GB/s); wall {dwall * 1e6 / nsteps:.1f} us/step")

    if args.copy_probe_mib > 0:
        # an elementwise kernel that reads and writes exactly n bytes each
        n = args.copy_probe_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe {args.copy_probe_mib} MiB x3 done")

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (float64 oracle)")
        result["cpu_baseline"] = cpu_baseline(cfg, x, min(args.cpu_baseline_tokens, T))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
