#!/usr/bin/env python3
"""Liger Attention throughput on one MI355X.

A step is one prefill of the Llama-3-8B-shaped workload
(B=1, T=8192, H_q=32, H_kv=8, d=128, bf16, scalar gate, window 64,
alpha 0.5) with its inputs already resident in device memory. Each timed
step is one call of the library (its three kernels back to back)
bracketed by HIP events on the stream the kernels run on; the output
kernel's own duration comes from steps of their own in which an event
separates it from the first two kernels. Before
each one an untimed 1 GiB read evicts the step's data from the 256 MB
last-level cache, so the inputs come from HBM ("cold", the headline
`value`, median step). The same steps without the eviction are reported as
"hot", and steps after a 512 MiB write instead (whose dirty lines are
written back during the step) as "cold_write_evicted". The JSON line also
carries:
  - the roofline of the dominant kernel (the fused output kernel) and the
    whole cold step's fraction of the same roofline;
  - the other prefill workloads, each with its own roofline: the
    Llama-3.2-1B-shaped batch (B=4, T=2048, d=64, vector gate) and the
    long-context 8B shape (T=32768, vector gate, 1% of key rows x8);
  - the decode workload (64 sequences, Llama-3-8B heads, 1024 single-token
    steps: launched back to back, each between its own events, replayed from
    a captured HIP graph, and cold steps after evicting the cache);
  - the hybrid's full causal softmax attention layer, the prefill with sink
    tokens, and the prefill's backward, on the 8B inputs;
  - the float64 CPU oracle on the host as a reported baseline (prefill of
    the 8B, 1B and long-context workloads and decode steps, each on a
    bounded sample), with the CPU model and thread counts.

    python bench.py [--steps K] [--warmup W] [--decode-steps N]

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector or MFMA)
PREFILL_WORKLOAD = "prefill_8b_b1_t8192_d128"
PREFILL_1B_WORKLOAD = "prefill_1b_b4_t2048_d64"
PREFILL_LONG_WORKLOAD = "prefill_8b_b1_t32768_d128_outliers"
OUTPUT_KERNEL_RECORD = {PREFILL_WORKLOAD: "prefill_output_kernel",
                        PREFILL_1B_WORKLOAD: "prefill_output_kernel_vector_d64",
                        PREFILL_LONG_WORKLOAD: "prefill_output_kernel_vector_d128"}
DECODE_WORKLOAD = "decode_8b_n64_d128"
FULL_WORKLOAD = "full_attn_8b_b1_t8192_d128"
N_SINKS = 16      # meta-memory tokens per key/value head in the sink measurements (synthetic, N(0, 1))
SINK_SEED = 17  # the softmax layer on the prefill workload's inputs
BWD_SEED = 23   # upstream gradient of the backward measurement
CHUNK = 64
SCRUB_BYTES = 512 << 20        # larger than the 256 MB last-level cache
READ_EVICT_BYTES = 1 << 30     # read through before each cold step
DECODE_LAYERS = 8              # layers of decode state stepped in turn (8 x 48 MiB > 256 MB last-level cache)
# tokens of each other prefill workload that the CPU baseline times (a prefix:
# the oracle is linear in T, so the prefix rate is the workload's rate)
CPU_PREFIX_TOKENS = {PREFILL_1B_WORKLOAD: 512, PREFILL_LONG_WORKLOAD: 1024}
PREFILL_FP32_WORKLOAD = "prefill_fp32_b1_h2_t256_d64"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counter_record(kernel: str, workload: str) -> dict:
    """Committed counter readings for this kernel, if its sources are unchanged since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return {}
    from gated_linear_recurrent_amd.counters import KERNELS, source_sha
    if rec.get("workload") != workload or rec.get("source_sha256") != source_sha(KERNELS[kernel][2]):
        return {}
    return rec


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE), or None."""
    return counter_record(kernel, workload).get("hbm_bytes_per_launch")


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


def cpu_info() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, CPUs this
    process may use, and the BLAS thread pools the oracle's NumPy could use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    info = {"cpu_model": model, "cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["affinity_cpus"] = None
    try:
        from threadpoolctl import threadpool_info
        info["blas_pools"] = [{"api": p.get("internal_api"), "threads": p.get("num_threads")}
                              for p in threadpool_info()]
    except Exception:  # report what is available
        info["blas_pools"] = None
    return info


def _timed_runs(fn, min_seconds: float, max_runs: int) -> list:
    times = []
    while sum(times) < min_seconds and len(times) < max_runs:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return times


def cpu_baseline_prefill(name: str, x: dict, tokens: int, min_seconds: float, max_runs: int = 20) -> dict:
    """The float64 oracle as it stands on the first `tokens` tokens of a
    prefill workload (all batches and heads), BLAS limited to one thread, run
    repeatedly until about min_seconds of CPU work are timed; the value is the
    median rate over the runs (the oracle is linear in T, so a prefix rate is
    the workload's rate)."""
    import oracle
    from synth import CONFIGS
    from threadpoolctl import threadpool_limits
    cfg = CONFIGS[name]
    gate = 0 if cfg["gate"] == "scalar" else 1
    q, k, v = (x[n][:, :tokens] for n in ("q", "k", "v"))
    with threadpool_limits(limits=1):
        times = _timed_runs(lambda: oracle.prefill(q, k, v, gate, cfg["window"], cfg["alpha"]), min_seconds, max_runs)
    dt = sorted(times)[len(times) // 2]
    return {"value": cfg["B"] * tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{name}: first {tokens} of {cfg['T']} tokens (all {cfg['B']} sequences and heads), "
                      f"float64 token loop, BLAS limited to 1 thread; {len(times)} runs, {sum(times):.1f} s "
                      f"in all, median {dt:.2f} s per run"}


def cpu_baseline_decode(name: str, steps: int, min_seconds: float, max_runs: int = 20) -> dict:
    """The float64 oracle's decode step over the first `steps` steps of the
    decode workload (all sequences), BLAS limited to one thread; steps/s is
    the median over repeated runs (inputs generated before the timing)."""
    import oracle
    from synth import CONFIGS, decode_initial, decode_step_inputs
    from threadpoolctl import threadpool_limits
    cfg = CONFIGS[name]
    gate = 0 if cfg["gate"] == "scalar" else 1
    init = decode_initial(**cfg)
    xs = [decode_step_inputs(step=s, **cfg) for s in range(steps)]

    def run():
        S, rk, rv, pos = init["S"], init["ring_k"], init["ring_v"], init["pos"]
        for x in xs:
            _, S, rk, rv, pos = oracle.decode_step(x["q"], x["k"], x["v"], S, rk, rv, pos, gate, cfg["alpha"])

    with threadpool_limits(limits=1):
        times = _timed_runs(run, min_seconds, max_runs)
    dt = sorted(times)[len(times) // 2]
    return {"value": steps / dt, "unit": "steps/s", "tokens_per_s": cfg["N"] * steps / dt, "cores": 1,
            "kind": "oracle",
            "sample": f"{name}: first {steps} of {cfg['steps']} steps, all {cfg['N']} sequences, float64, "
                      f"BLAS limited to 1 thread; {len(times)} runs, {sum(times):.1f} s in all, "
                      f"median {dt:.2f} s per run"}


class Evictor:
    """Empties the 256 MB last-level cache of the step's data before a cold step.

    "read" (the default, used for every cold figure): sums a 1 GiB buffer, so
    the cache is left holding clean lines of that buffer and the step's
    inputs come from HBM. "write": fills a 512 MiB buffer, so the cache is left
    full of dirty lines whose write-back to HBM then competes with the step;
    reported beside the read-evicted figures for the prefill and decode
    workloads, labelled."""

    def __init__(self, dev):
        import torch
        self.rbuf = torch.ones(READ_EVICT_BYTES // 4, dtype=torch.float32, device=dev)
        self.acc = torch.zeros((), dtype=torch.float32, device=dev)
        self.wbuf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
        self.device = dev

    def __call__(self, i: int, kind: str = "read"):
        import torch
        if kind == "read":
            torch.sum(self.rbuf, dim=(0,), out=self.acc)
        else:
            self.wbuf.fill_(float(i))


def stats(a) -> dict:
    import numpy as np
    return {"median_ms": float(np.median(a)), "min_ms": float(np.min(a)), "mean_ms": float(np.mean(a))}


def measure_prefill(name: str, x: dict, steps: int, warmup: int, scrub, log_tag: str) -> dict:
    """Cold and hot prefill steps of a named workload. Each step is two
    enqueues on one stream (segment states + carry scan, then the output
    kernel), bracketed by three HIP events, so the output kernel's launch
    duration is measured on the stream it runs on. Returns the step times,
    tokens/s at the cold median, and the roofline of the output kernel."""
    import numpy as np
    import torch

    import gated_linear_recurrent_amd as gla
    from synth import CONFIGS
    cfg = CONFIGS[name]
    dev = scrub.device
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt).contiguous() for n in ("q", "k", "v"))
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    gate = gla.LIGER_GATE_SCALAR_MEAN if cfg["gate"] == "scalar" else gla.LIGER_GATE_VECTOR_AVGPOOL4
    o = torch.empty_like(q)
    S_T = torch.empty((B, H_kv, d, d), dtype=torch.float32, device=dev)
    code = gla.LIGER_BF16 if cfg["dtype"] == "bf16" else gla.LIGER_F32
    ws = torch.empty(max(gla.liger_attn_prefill_workspace_size(B, T, H_q, H_kv, d, code), 16),
                     dtype=torch.uint8, device=dev)

    def prefill(mask):
        gla.liger_attn_prefill(q, k, v, gate, cfg["window"], cfg["alpha"], o=o, S_T=S_T, workspace=ws,
                               stage_mask=mask)

    def timed(n: int, cold, kind: str = "read"):
        """Per step, the stages enqueued by two calls with an event between them:
        (segment states + carry scan, output kernel, total) in ms."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i, e in enumerate(ev):
            if cold:
                scrub(i, kind)
            e[0].record()
            prefill(gla.LIGER_STAGE_SEGMENT_STATES | gla.LIGER_STAGE_CARRY_SCAN)
            e[1].record()
            prefill(gla.LIGER_STAGE_OUTPUT)
            e[2].record()
        torch.cuda.synchronize()
        return np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[0].elapsed_time(e[2])] for e in ev])

    def timed_whole(n: int, cold, kind: str = "read"):
        """Per step, one call (all three kernels back to back) between two events, in ms."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for i, e in enumerate(ev):
            if cold:
                scrub(i, kind)
            e[0].record()
            prefill(7)
            e[1].record()
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in ev])

    log(f"[bench] {log_tag}: warmup {warmup}, then {steps} cold + {steps} hot steps")
    for _ in range(warmup):
        prefill(7)
    torch.cuda.synchronize()
    # The step is one call; the event a split between the stages needs costs
    # about 5 us (the output kernel then starts that much after the carry
    # scan ends), so the stage split runs in steps of its own.
    cold_whole = timed_whole(steps, True)
    hot_whole = timed_whole(steps, False)
    cold = timed(steps, True)
    hot = timed(steps, False)
    cold_w = timed(max(5, steps // 2), True, "write")
    cold_w_whole = timed_whole(max(5, steps // 2), True, "write")
    ms_cold = float(np.median(cold_whole))
    byts, flops = prefill_algorithmic(cfg)
    # the dominant kernel's average launch duration over every timed launch
    out_ms = float(np.mean(np.concatenate([cold[:, 1], hot[:, 1]])))
    achieved = byts / (out_ms * 1e-3) / 1e9
    kname = OUTPUT_KERNEL_RECORD[name]
    crec = counter_record(kname, name)
    traffic = crec.get("hbm_bytes_per_launch")
    peak_mfma = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS
    log(f"[bench] {log_tag}: cold {ms_cold * 1e3:.1f} us/step (hot {np.median(hot_whole) * 1e3:.1f}); "
        f"output kernel {out_ms * 1e3:.1f} us ({achieved:.0f} GB/s); "
        f"segment states + carry scan cold {np.median(cold[:, 0]) * 1e3:.1f} us")
    return {
        "workload": name, "B": B, "T": T, "H_q": H_q, "H_kv": H_kv, "d": d, "gate": cfg["gate"],
        "window": cfg["window"], "alpha": cfg["alpha"], "steps": steps, "warmup": warmup,
        "ms_per_step_cold": ms_cold,
        "tokens_per_s": B * T / (ms_cold * 1e-3),
        "tokens_per_s_hot": B * T / (float(np.median(hot_whole)) * 1e-3),
        "cold": {"total": stats(cold_whole), "segment_states_and_carry_scan": stats(cold[:, 0]),
                 "output": stats(cold[:, 1]), "total_with_stage_event": stats(cold[:, 2])},
        "hot": {"total": stats(hot_whole), "segment_states_and_carry_scan": stats(hot[:, 0]),
                "output": stats(hot[:, 1]), "total_with_stage_event": stats(hot[:, 2])},
        "cold_write_evicted": {"total": stats(cold_w_whole), "output": stats(cold_w[:, 1]),
                               "note": "cache emptied by a 512 MiB write: its dirty lines are written back "
                                       "during the step"},
        # whole cold step against the same (HBM) roofline as the kernel below
        "step_roofline_frac": byts / (ms_cold * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kname, "kernel_ms": out_ms,
                     "algorithmic_bytes": byts, "algorithmic_flops": flops,
                     "mfma_frac_algorithmic": flops / (out_ms * 1e-3) / (peak_mfma * 1e12),
                     "mfma_busy_frac_counters": crec.get("mfma_busy_frac"),
                     "valu_busy_frac_counters": crec.get("valu_busy_frac"),
                     "lds_bank_conflict_frac_counters": crec.get("lds_bank_conflict_frac"),
                     "tcc_ea_gbs_counters": (traffic / (out_ms * 1e-3) / 1e9) if traffic else None},
    }, (q, k, v, o, S_T, ws, gate)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-full", action="store_true", help="skip the full causal attention layer")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy and GEMM peaks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the 1B-shaped and long-context prefill workloads")
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
    scrub = Evictor(dev)
    cfg = CONFIGS[PREFILL_WORKLOAD]
    log(f"[bench] generating {PREFILL_WORKLOAD}")
    x = config_prefill_inputs(PREFILL_WORKLOAD)
    head, bufs = measure_prefill(PREFILL_WORKLOAD, x, args.steps, args.warmup, scrub, "prefill 8B T=8192")
    q, k, v, o, S_T, ws, gate = bufs
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    ms_per_step = head["ms_per_step_cold"]

    result = {
        "metric": "Liger Attention prefill tokens/s/GPU at 8B shapes; decode steps/s; % roofline",
        "value": head["tokens_per_s"],
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
        "roofline": dict(head["roofline"], step_frac=head["step_roofline_frac"]),
        "prefill_cold": head["cold"],
        "prefill_hot": dict(head["hot"], tokens_per_s=head["tokens_per_s_hot"]),
        "prefill_op_roofline_frac": head["step_roofline_frac"],
    }

    # the other prefill workloads, each with its own roofline
    cpu_prefix = {}  # the prefixes the CPU baseline times, kept from the same draws
    if not args.no_other_prefill:
        others = {}
        for name, tag in ((PREFILL_1B_WORKLOAD, "prefill 1B B=4 T=2048"),
                          (PREFILL_LONG_WORKLOAD, "prefill 8B T=32768 outliers")):
            log(f"[bench] generating {name}")
            xo = config_prefill_inputs(name)
            others[name], _ = measure_prefill(name, xo, max(5, args.steps // 2), max(2, args.warmup // 2), scrub, tag)
            cpu_prefix[name] = {n: np.ascontiguousarray(xo[n][:, :CPU_PREFIX_TOKENS[name]]) for n in ("q", "k", "v")}
            del xo
            torch.cuda.empty_cache()
        result["prefill_other_workloads"] = others

    if not args.no_full:
        # the hybrid's softmax layer on the same 8B inputs (q, k, v in HBM)
        fo = torch.empty_like(q)
        for _ in range(max(1, args.warmup // 2)):
            gla.liger_attn_full_causal(q, k, v, o=fo)
        torch.cuda.synchronize()
        nfull = max(5, args.steps // 2)

        def timed_full(cold_steps: bool):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nfull)]
            for i, (e0, e1) in enumerate(ev):
                if cold_steps:
                    scrub(i)
                e0.record()
                gla.liger_attn_full_causal(q, k, v, o=fo)
                e1.record()
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in ev])

        fcold, fhot = timed_full(True), timed_full(False)
        fflops = 4.0 * d * (T * (T + 1) / 2) * H_q * B  # q.k and p.v over the causal pairs
        fms = float(np.mean(np.concatenate([fcold, fhot])))
        fach = fflops / (fms * 1e-3) / 1e12
        frec = counter_record("full_attn_kernel", FULL_WORKLOAD)
        result["full_attention"] = {
            "workload": FULL_WORKLOAD, "steps": nfull,
            "cold": stats(fcold), "hot": stats(fhot),
            "tokens_per_s": B * T / (float(np.median(fcold)) * 1e-3),
            "roofline": {"bound": "mfma", "achieved": fach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": fach / PEAK_BF16_TFLOPS, "traffic": frec.get("hbm_bytes_per_launch"),
                         "kernel": "full_attn_kernel", "kernel_ms": fms, "algorithmic_flops": fflops,
                         "mfma_busy_frac_counters": frec.get("mfma_busy_frac")},
        }
        log(f"[bench] full attention {fms * 1e3:.1f} us ({fach:.0f} TFLOP/s, "
            f"{100 * fach / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")

    # the same prefill with meta-memory sink tokens prepended to every window
    rng = np.random.default_rng(SINK_SEED)
    sink_np = [rng.standard_normal((H_kv, N_SINKS, d)).astype(np.float32) for _ in range(2)]
    psinks = tuple(torch.from_numpy(a).to(dev).to(torch.bfloat16) for a in sink_np)

    def prefill_sinks():
        gla.liger_attn_prefill(q, k, v, gate, cfg["window"], cfg["alpha"], o=o, S_T=S_T, workspace=ws, sinks=psinks)

    for _ in range(max(1, args.warmup // 2)):
        prefill_sinks()
    torch.cuda.synchronize()

    def timed_sinks(cold_steps: bool):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i, (e0, e1) in enumerate(ev):
            if cold_steps:
                scrub(i)
            e0.record()
            prefill_sinks()
            e1.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    scold, shot = timed_sinks(True), timed_sinks(False)
    result["prefill_sinks"] = {"workload": PREFILL_WORKLOAD, "n_sinks": N_SINKS, "cold": stats(scold), "hot": stats(shot),
                               "tokens_per_s": B * T / (float(np.median(scold)) * 1e-3)}
    log(f"[bench] prefill with {N_SINKS} sinks: cold {np.median(scold) * 1e3:.1f} us, hot {np.median(shot) * 1e3:.1f} us")

    if not args.no_backward:
        # the prefill's backward on the same inputs, upstream gradient dO ~ N(0, 1) (bf16)
        from synth import grad_output
        dO = torch.from_numpy(grad_output(x["q"].shape, "bf16", seed=BWD_SEED)).to(dev).to(torch.bfloat16)
        bdq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        bdk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        bdv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        bws = torch.empty(max(gla.liger_attn_prefill_backward_workspace_size(B, T, H_q, H_kv, d), 16),
                          dtype=torch.uint8, device=dev)

        def backward():
            gla.liger_attn_prefill_backward(q, k, v, dO, gate, cfg["window"], cfg["alpha"], dq=bdq, dk=bdk, dv=bdv,
                                            workspace=bws)

        for _ in range(max(1, args.warmup // 2)):
            backward()
        torch.cuda.synchronize()
        nb = max(5, args.steps // 2)

        def timed_backward(cold_steps: bool):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb)]
            for i, (e0, e1) in enumerate(ev):
                if cold_steps:
                    scrub(i)
                e0.record()
                backward()
                e1.record()
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in ev])

        bcold, bhot = timed_backward(True), timed_backward(False)
        result["backward"] = {"workload": PREFILL_WORKLOAD, "steps": nb, "cold": stats(bcold), "hot": stats(bhot),
                              "tokens_per_s": B * T / (float(np.median(bcold)) * 1e-3),
                              "vs_forward_cold": float(np.median(bcold)) / ms_per_step,
                              "workspace_bytes": int(bws.numel())}
        log(f"[bench] backward cold {np.median(bcold) * 1e3:.1f} us, hot {np.median(bhot) * 1e3:.1f} us")

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

        def dstep(s):
            gla.liger_attn_decode_step(*steps_in[s], S, ring, dgate, dcfg["alpha"], o=do)

        dwarm = min(16, nsteps)
        for s in range(dwarm):
            dstep(s)
        torch.cuda.synchronize()
        # the timed region: nsteps launches back to back between one pair of
        # events; the average launch duration is its length over nsteps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for s in range(nsteps):
            dstep(s)
        e1.record()
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        k_ms = e0.elapsed_time(e1) / nsteps
        # the same launches, each between its own pair of events (the events
        # add their own time to each launch)
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
        for s in range(nsteps):
            dev_ev[s][0].record()
            dstep(s)
            dev_ev[s][1].record()
        torch.cuda.synchronize()
        k_all = np.array([a.elapsed_time(b) for a, b in dev_ev])
        # the same launches replayed from one captured graph (no host work per step)
        glen = min(64, nsteps)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for s in range(glen):
                    dstep(s)
        torch.cuda.current_stream().wait_stream(cap)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, nsteps // glen)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / (reps * glen)
        # cold steps: the last-level cache is evicted before each one (read
        # eviction; write eviction reported beside it), each step between its
        # own pair of events like per_launch_events_us
        ncold = min(32, nsteps)

        def timed_cold(kind: str) -> float:
            cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(ncold)]
            for s in range(ncold):
                scrub(s, kind)
                cold_ev[s][0].record()
                dstep(s)
                cold_ev[s][1].record()
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in cold_ev])) * 1e3

        cold_us = timed_cold("read")
        cold_w_us = timed_cold("write")
        # cold back to back, as in a multi-layer model: DECODE_LAYERS layers'
        # states (more than the last-level cache holds together) stepped in
        # turn, so each step finds its state evicted by the other layers' steps
        lstate = [(S, ring)]
        for _ in range(DECODE_LAYERS - 1):
            lstate.append((S.clone(), gla.KVRing(ring.k.clone(), ring.v.clone(), ring.pos.clone(),
                                                 torch.zeros(N, dtype=torch.int32, device=dev), w)))

        def lstep(s):
            Sl, rl = lstate[s % DECODE_LAYERS]
            gla.liger_attn_decode_step(*steps_in[s], Sl, rl, dgate, dcfg["alpha"], o=do)

        for s in range(2 * DECODE_LAYERS):
            lstep(s)
        torch.cuda.synchronize()
        e0.record()
        for s in range(nsteps):
            lstep(s)
        e1.record()
        torch.cuda.synchronize()
        multi_us = e0.elapsed_time(e1) * 1e3 / nsteps
        del lstate
        # the same steps with meta-memory sink tokens, back to back
        rng = np.random.default_rng(SINK_SEED + 1)
        dsinks = tuple(torch.from_numpy(rng.standard_normal((Hkv, N_SINKS, dd)).astype(np.float32)).to(dev)
                       .to(torch.bfloat16) for _ in range(2))
        for s in range(dwarm):
            gla.liger_attn_decode_step(*steps_in[s], S, ring, dgate, dcfg["alpha"], o=do, sinks=dsinks)
        e0.record()
        for s in range(nsteps):
            gla.liger_attn_decode_step(*steps_in[s], S, ring, dgate, dcfg["alpha"], o=do, sinks=dsinks)
        e1.record()
        torch.cuda.synchronize()
        sink_us = e0.elapsed_time(e1) * 1e3 / nsteps
        dbytes = decode_algorithmic(dcfg)
        dach = dbytes / (k_ms * 1e-3) / 1e9
        drec = counter_record("decode_step_kernel", DECODE_WORKLOAD)
        dtraffic = drec.get("hbm_bytes_per_launch")
        result["decode"] = {
            "workload": DECODE_WORKLOAD, "steps": nsteps, "warmup": dwarm,
            "steps_per_s": nsteps / dwall, "us_per_step_wall": dwall * 1e6 / nsteps,
            "kernel_us": k_ms * 1e3, "per_launch_events_us_median": float(np.median(k_all)) * 1e3,
            "per_launch_events_us_min": float(np.min(k_all)) * 1e3,
            "steps_per_s_kernel": 1e3 / k_ms, "tokens_per_s_kernel": N * 1e3 / k_ms,
            "graph_us_per_step": graph_us, "graph_steps_per_s": 1e6 / graph_us,
            "cold_kernel_us_median": cold_us,
            "cold_write_evicted_us_median": cold_w_us,
            "cold_multilayer_us": multi_us, "multilayer_layers": DECODE_LAYERS,
            "with_sinks": {"n_sinks": N_SINKS, "kernel_us": sink_us},
            "roofline": {"bound": "hbm", "achieved": dach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": dach / PEAK_HBM_GBS, "traffic": dtraffic,
                         "regime": "hot: back-to-back steps, the 48 MiB state + ring working set "
                                   "stays in the 256 MB last-level cache",
                         "cold_frac": dbytes / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                         "cold_multilayer_frac": dbytes / (multi_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                         "cold_regime": "cold: median of single steps, each between its own events (which add "
                                        "about what per_launch_events_us adds to kernel_us), after evicting the "
                                        "last-level cache with a 1 GiB read (as in a multi-layer model, where "
                                        "each layer's state is evicted between steps); after a 512 MiB write "
                                        "instead, the dirty lines' write-back adds to the step: "
                                        "cold_write_evicted_us_median; cold_multilayer: steps back to back "
                                        "over the states of several layers (384 MiB together), each layer's "
                                        "state evicted by the others' steps",
                         "kernel": "decode_step_kernel", "algorithmic_bytes": dbytes,
                         "tcc_ea_gbs_counters": (dtraffic / (k_ms * 1e-3) / 1e9) if dtraffic else None,
                         "counters_by_regime": drec.get("regimes")},
        }
        log(f"[bench] decode kernel {k_ms * 1e3:.1f} us/step ({dach:.0f} GB/s); graph {graph_us:.1f} us/step; "
            f"cold {cold_us:.1f} us (write-evicted {cold_w_us:.1f}; {DECODE_LAYERS} layers back to back "
            f"{multi_us:.1f}); wall {dwall * 1e6 / nsteps:.1f} us/step")

    if not args.no_peaks:
        # what the box reaches with plain library work, next to the datasheet peaks:
        # a device-to-device copy of 1 GiB (read + write) and a bf16 GEMM (hipBLASLt) of 8192^3
        n = 1 << 28
        a = torch.empty(n, dtype=torch.float32, device=dev)
        c = torch.empty_like(a)
        for _ in range(3):
            c.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            c.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * n * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del a, c
        m = 8192
        ga = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
        gb = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            gc = torch.matmul(ga, gb)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            gc = torch.matmul(ga, gb)
        e1.record()
        torch.cuda.synchronize()
        gemm_tflops = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        del ga, gb, gc
        result["measured_peaks"] = {"copy_gbs": copy_gbs, "bf16_gemm_tflops": gemm_tflops,
                                    "note": "1 GiB fp32 device copy (read + write); 8192^3 bf16 torch.matmul"}
        result["roofline"]["frac_of_measured_copy"] = result["roofline"]["achieved"] / copy_gbs
        if "decode" in result:
            result["decode"]["roofline"]["frac_of_measured_copy"] = result["decode"]["roofline"]["achieved"] / copy_gbs
        if "full_attention" in result:
            fr = result["full_attention"]["roofline"]
            fr["frac_of_measured_gemm"] = fr["achieved"] / gemm_tflops
        log(f"[bench] measured peaks: copy {copy_gbs:.0f} GB/s, bf16 GEMM {gemm_tflops:.0f} TFLOP/s")

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
        # the oracle as it stands, on bounded samples of each workload (about
        # 20 s of CPU work in all); GPU rates beside it for the ratio
        log("[bench] cpu baseline (float64 oracle)")
        cb = cpu_baseline_prefill(PREFILL_WORKLOAD, x, min(args.cpu_baseline_tokens, T), min_seconds=8.0)
        cb["gpu_over_oracle"] = result["value"] / cb["value"]
        cb["host"] = cpu_info()
        legs = {}
        for name in (PREFILL_1B_WORKLOAD, PREFILL_LONG_WORKLOAD):
            xp = cpu_prefix.get(name) or config_prefill_inputs(name, T=CPU_PREFIX_TOKENS[name])
            legs[name] = cpu_baseline_prefill(name, xp, CPU_PREFIX_TOKENS[name], min_seconds=4.0)
        legs[DECODE_WORKLOAD] = cpu_baseline_decode(DECODE_WORKLOAD, 16, min_seconds=4.0)
        # the small fp32 workload (a correctness case, not timed on the GPU), whole
        legs[PREFILL_FP32_WORKLOAD] = cpu_baseline_prefill(PREFILL_FP32_WORKLOAD,
                                                           config_prefill_inputs(PREFILL_FP32_WORKLOAD),
                                                           CONFIGS[PREFILL_FP32_WORKLOAD]["T"], min_seconds=1.0)
        other = result.get("prefill_other_workloads", {})
        for name, leg in legs.items():
            if name in other:
                leg["gpu_over_oracle"] = other[name]["tokens_per_s"] / leg["value"]
        if "decode" in result:
            legs[DECODE_WORKLOAD]["gpu_over_oracle"] = result["decode"]["steps_per_s_kernel"] / legs[DECODE_WORKLOAD]["value"]
        cb["other_workloads"] = legs
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
