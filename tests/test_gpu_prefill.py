"""GPU parity of liger_attn_prefill against the float64 oracle.

Every case prints its name before touching the GPU. Inputs are seeded
(synth/), the oracle runs on the same canonical values, and the parity bars
are those of tests/liger_testutil.py.
"""
import numpy as np
import pytest
import torch

import oracle
from liger_testutil import check_prefill, gpu_prefill, say, to_np
from synth import CONFIGS, GATE_MODES, config_prefill_inputs, prefill_inputs, round_to_bf16

pytestmark = pytest.mark.gpu


def _run_case(x, dtype, gate, window, alpha=0.5, cps=0, tag=""):
    say(f"[prefill] {tag} dtype={dtype} gate={gate} window={window} alpha={alpha} cps={cps} "
        f"q={x['q'].shape} k={x['k'].shape}")
    o_ref, S_ref, o_grm, _ = oracle.prefill(x["q"], x["k"], x["v"], gate, window, alpha, return_parts=True)
    o, S = gpu_prefill(x, dtype, gate, window, alpha, cps)
    o1, _ = gpu_prefill(x, dtype, gate, window, 1.0, cps)
    return check_prefill(dtype, to_np(o), o_ref, to_np(S), S_ref, to_np(o1), o_grm, tag=tag)


def test_library_is_native():
    """The HIP library is what runs: loaded from the package directory."""
    import gated_linear_recurrent_amd as gla
    lib = gla.load_library()
    assert lib._name == gla.LIB_PATH
    assert torch.cuda.is_available()


@pytest.mark.parametrize("cps", [0, 1])
def test_config_fp32_small(cps):
    name = "prefill_fp32_b1_h2_t256_d64"
    cfg = CONFIGS[name]
    x = config_prefill_inputs(name)
    _run_case(x, cfg["dtype"], GATE_MODES[cfg["gate"]], cfg["window"], cfg["alpha"], cps, tag=name)


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("n_rep", [1, 4])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 100])
@pytest.mark.parametrize("window", [1, 17, 64])
def test_fp32_edges(gate, n_rep, T, window):
    x = prefill_inputs(B=2, T=T, H_q=2 * n_rep, H_kv=2, d=64, dtype="f32", seed=T * 7 + window)
    _run_case(x, "f32", gate, window, 0.5, cps=1, tag=f"fp32 T={T} w={window} n_rep={n_rep}")


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("n_rep", [1, 4])
@pytest.mark.parametrize("T,cps", [(1, 0), (64, 0), (65, 1), (200, 0), (200, 1), (450, 3)])
@pytest.mark.parametrize("window", [1, 17, 64])
def test_fp32_d128(gate, n_rep, T, cps, window):
    """fp32 at d = 128: the window halo and the state operand come from global
    memory, and the output kernel also writes the segment records."""
    x = prefill_inputs(B=2, T=T, H_q=2 * n_rep, H_kv=2, d=128, dtype="f32", seed=T * 11 + window + n_rep)
    _run_case(x, "f32", gate, window, 0.5, cps=cps, tag=f"fp32 d=128 T={T} w={window} n_rep={n_rep} cps={cps}")


@pytest.mark.parametrize("gate", [0, 1])
def test_fp32_d128_eight_query_heads_per_kv_head(gate):
    """Sixteen output blocks per chunk for eight waves, three sequences."""
    x = prefill_inputs(B=3, T=260, H_q=8, H_kv=1, d=128, dtype="f32", seed=91 + gate)
    _run_case(x, "f32", gate, 64, 0.5, cps=1, tag=f"fp32 d=128 n_rep=8 gate={gate}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("T,n_rep,cps", [(1, 4, 0), (100, 1, 0), (300, 4, 1), (513, 4, 2), (1000, 2, 0)])
def test_bf16_shapes(d, gate, T, n_rep, cps):
    x = prefill_inputs(B=2, T=T, H_q=2 * n_rep, H_kv=2, d=d, dtype="bf16", seed=T + d)
    _run_case(x, "bf16", gate, 64, 0.5, cps, tag=f"bf16 d={d} T={T} n_rep={n_rep}")


@pytest.mark.parametrize("window,alpha", [(17, 0.25), (1, 0.9), (64, 0.0), (64, 1.0)])
def test_bf16_window_and_alpha(window, alpha):
    x = prefill_inputs(B=1, T=333, H_q=8, H_kv=2, d=128, dtype="bf16", seed=window)
    _run_case(x, "bf16", 1, window, alpha, 0, tag=f"bf16 w={window} alpha={alpha}")


def _strong_decay_keys(x, rng, d):
    """Channel groups whose pooled gate is tiny (decay ~2^-20 per token) while
    the middle channel dominates phi(k): the MFMA factorisation of those
    channels would overflow, so they take the exact path."""
    k = x["k"]
    for c in rng.choice(np.arange(2, d - 3), size=3, replace=False):
        k[..., c - 1] = -20.0
        k[..., c] = 6.0
        k[..., c + 1] = -20.0
        k[..., c + 2] = -20.0
    return x


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_vector_gate_extreme_decay_channels(dtype, d):
    rng = np.random.default_rng(3)
    x = prefill_inputs(B=1, T=200, H_q=4, H_kv=1, d=d, dtype=dtype, seed=17)
    x = _strong_decay_keys(x, rng, d)
    _run_case(x, dtype, 1, 64, 0.5, 1, tag=f"extreme vector decay {dtype} d={d}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 128)])
def test_scalar_gate_extreme_decay(dtype, d):
    x = prefill_inputs(B=1, T=200, H_q=4, H_kv=1, d=d, dtype=dtype, seed=19)
    x["k"][:, 50:120] -= 30.0   # mean key ~ -30: gate ~ e^-30 on these tokens
    if dtype == "bf16":         # keep the canonical inputs bf16-exact on both sides
        x["k"] = round_to_bf16(x["k"])
    _run_case(x, dtype, 0, 64, 0.5, 1, tag=f"extreme scalar decay {dtype}")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("cps", [1, 3, 10])
def test_slow_decay_across_segments(dtype, d, gate, cps):
    """Keys shifted by +6: phi(k) is unchanged (a softmax over the channels)
    while every gate becomes sigma(~6) ~ 0.9975, so the state keeps hundreds
    of tokens and the chunk-to-chunk, block-to-block and segment-to-segment
    decays all reach the output (T = 640: ten chunks in segments of 1, 3 or
    10 chunks)."""
    x = prefill_inputs(B=1, T=640, H_q=4, H_kv=1, d=d, dtype=dtype, seed=23 + d + gate)
    x["k"] = x["k"] + 6.0
    if dtype == "bf16":  # keep the canonical inputs bf16-exact on both sides
        x["k"] = round_to_bf16(x["k"])
    _run_case(x, dtype, gate, 64, 0.5, cps, tag=f"slow decay {dtype} d={d} gate={gate} cps={cps}")


def test_deterministic_and_fully_written():
    x = prefill_inputs(B=1, T=700, H_q=8, H_kv=2, d=128, dtype="bf16", seed=5)
    say("[prefill] determinism bf16 d=128 T=700")
    o1, S1 = gpu_prefill(x, "bf16", 1, 64, 0.5, 2)
    o2, S2 = gpu_prefill(x, "bf16", 1, 64, 0.5, 2)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert bool(torch.isfinite(o1.float()).all()) and bool(torch.isfinite(S1).all())


def test_segmentation_invariance():
    x = prefill_inputs(B=1, T=640, H_q=4, H_kv=1, d=128, dtype="bf16", seed=8)
    say("[prefill] segment lengths 1, 2, 3, 10 on T=640")
    outs = [gpu_prefill(x, "bf16", 1, 64, 0.5, cps) for cps in (1, 2, 3, 10)]
    o_ref, S_ref = oracle.prefill(x["q"], x["k"], x["v"], 1, 64, 0.5)
    for o, S in outs:
        check_prefill("bf16", to_np(o), o_ref, to_np(S), S_ref, tag="segmentation")
    for o, S in outs[1:]:
        assert float((o.float() - outs[0][0].float()).abs().max()) <= 2e-2
        assert float((S - outs[0][1]).abs().max()) <= 1e-3 * float(outs[0][1].abs().max())


@pytest.mark.parametrize("name", ["prefill_1b_b4_t2048_d64", "prefill_8b_b1_t8192_d128",
                                  "prefill_8b_b1_t32768_d128_outliers"])
def test_config_full_size(name):
    """The named workloads at their full sizes, in the default launch plan."""
    cfg = CONFIGS[name]
    x = config_prefill_inputs(name)
    _run_case(x, cfg["dtype"], GATE_MODES[cfg["gate"]], cfg["window"], cfg["alpha"], 0, tag=name)
