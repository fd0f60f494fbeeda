"""GPU parity of the prefill backward (dq, dk, dv of sum(o * dO)) against the
float64 oracle's reverse pass, on bf16 inputs (the gradients are float32).

Bar: for each of dq, dk, dv, max |gpu - ref| <= 1e-4 * max |ref| (the
fp32 bar of the forward). Every product is fp32-accurate (raw bf16 operands
exactly, computed operands as hi + lo bf16 pairs with a residual below
2^-17), so the errors come from fp32 rounding, the split residual and the
hardware exp2 (measured: at most 1.6e-5 of max |ref|).

Cases span one and many 64-token chunks, ragged tails, T = 1 up to the
full 8B shape (T = 8192, 32 query heads) and the full 1B shape (B = 4,
T = 2048, d = 64, vector gate), windows 1 .. 64, H_q / H_kv
from 1 to 8, alpha = 0 and 1, both gates, and keys
scaled x40 so that gate channels become extreme (cumulative decay beyond
2^96 inside a chunk: the pair-by-pair path).
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrent_amd as gla
import oracle
from liger_testutil import DEV, say, to_dev, to_np
from synth import grad_output, prefill_inputs, round_to_bf16

pytestmark = pytest.mark.gpu

BAR = 1e-4


def _run(x, dO, gate, window, alpha):
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    g = to_dev(dO, "bf16")
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full(v.shape, float("nan"), dtype=torch.float32, device=DEV)
    gla.liger_attn_prefill_backward(q, k, v, g, gate, window, alpha, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv)


def _check(got, ref, tag):
    errs = []
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(a)), f"{tag}: {name} has non-finite entries"
        scale = max(float(np.max(np.abs(r))), 1e-30)
        errs.append(float(np.max(np.abs(a - r))) / scale)
    say(f"  {tag}: rel err dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    assert max(errs) <= BAR, (tag, errs)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("B,T,n_rep,window", [(2, 100, 1, 64), (1, 300, 4, 64), (2, 130, 2, 7),
                                              (1, 70, 8, 1), (1, 64, 4, 33), (1, 1, 2, 64), (1, 128, 3, 64)])
def test_backward_matches_oracle(d, gate, B, T, n_rep, window):
    H_kv = 2
    tag = f"bwd d={d} gate={gate} B={B} T={T} n_rep={n_rep} w={window}"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=B, T=T, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=T + 3 * n_rep + d + gate)
    dO = grad_output(x["q"].shape, "bf16", seed=T + window)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, gate, window, 0.5)
    _check(_run(x, dO, gate, window, 0.5), ref, tag)


@pytest.mark.parametrize("alpha", [0.0, 1.0])
@pytest.mark.parametrize("gate", [0, 1])
def test_backward_alpha_ends(alpha, gate):
    tag = f"bwd alpha={alpha} gate={gate}"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=1, T=200, H_q=8, H_kv=2, d=128, dtype="bf16", seed=17 + gate)
    dO = grad_output(x["q"].shape, "bf16", seed=23)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, gate, 64, alpha)
    _check(_run(x, dO, gate, 64, alpha), ref, tag)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_extreme_gate_channels(d):
    """Keys x40: per-channel decays beyond 2^96 within a chunk (vector gate)."""
    tag = f"bwd extreme d={d}"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=1, T=150, H_q=4, H_kv=2, d=d, dtype="bf16", seed=77)
    x["k"] = round_to_bf16(x["k"] * 40.0)
    dO = grad_output(x["q"].shape, "bf16", seed=5)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, 1, 64, 0.5)
    _check(_run(x, dO, 1, 64, 0.5), ref, tag)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", [0, 1])
def test_backward_slow_decay(d, gate):
    """Keys shifted by +6: phi(k) is unchanged and every gate is ~0.9975, so
    the chunk-start states and the adjoints flowing back from later tokens
    carry over hundreds of tokens through both scans (T = 400, alpha = 1:
    the recurrence alone)."""
    tag = f"bwd slow decay d={d} gate={gate}"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=1, T=400, H_q=8, H_kv=2, d=d, dtype="bf16", seed=401 + d + gate)
    x["k"] = round_to_bf16(x["k"] + 6.0)
    dO = grad_output(x["q"].shape, "bf16", seed=11)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, gate, 64, 1.0)
    _check(_run(x, dO, gate, 64, 1.0), ref, tag)


def test_backward_long_sequence():
    """32 chunks through both scans: T = 2048, H_q = 8, H_kv = 2, d = 128."""
    tag = "bwd long"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=1, T=2048, H_q=8, H_kv=2, d=128, dtype="bf16", seed=2048)
    dO = grad_output(x["q"].shape, "bf16", seed=9)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, 1, 64, 0.5)
    _check(_run(x, dO, 1, 64, 0.5), ref, tag)


@pytest.mark.timeout(600)
def test_backward_8b_shape_full():
    """The bench's backward workload in full: T = 8192, H_q = 32, H_kv = 8,
    d = 128, scalar gate, window 64, alpha 0.5, dO from seed 23; every
    element of dq, dk, dv against the float64 reverse pass (about a minute
    of host time, 11 GB of host memory)."""
    from synth import config_prefill_inputs
    x = config_prefill_inputs("prefill_8b_b1_t8192_d128")
    dO = grad_output(x["q"].shape, "bf16", seed=23)
    say("[bwd] 8B shape: GPU")
    got = _run(x, dO, 0, 64, 0.5)
    say("[bwd] 8B shape: oracle")
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, 0, 64, 0.5)
    _check(got, ref, "bwd 8B shape")


@pytest.mark.timeout(600)
def test_backward_1b_shape_full():
    """The 1B-shaped workload in full: B = 4, T = 2048, H_q = 32, H_kv = 8,
    d = 64, vector gate, window 64, alpha 0.5, dO from seed 29; every element
    of dq, dk, dv against the float64 reverse pass (about 15 s of host time,
    3.3 GB of host memory)."""
    from synth import config_prefill_inputs
    x = config_prefill_inputs("prefill_1b_b4_t2048_d64")
    dO = grad_output(x["q"].shape, "bf16", seed=29)
    say("[bwd] 1B shape: GPU")
    got = _run(x, dO, 1, 64, 0.5)
    say("[bwd] 1B shape: oracle")
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, 1, 64, 0.5)
    _check(got, ref, "bwd 1B shape")


def test_backward_outlier_keys():
    """The long-context recipe's key outliers (1% of key rows x8) with the
    vector gate at T = 1024, H_q = 8, H_kv = 2, d = 128."""
    tag = "bwd outlier keys"
    say(f"[bwd] {tag}")
    x = prefill_inputs(B=1, T=1024, H_q=8, H_kv=2, d=128, dtype="bf16", seed=55, outlier_frac=0.01,
                       outlier_scale=8.0)
    dO = grad_output(x["q"].shape, "bf16", seed=56)
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], dO, 1, 64, 0.5)
    _check(_run(x, dO, 1, 64, 0.5), ref, tag)


@pytest.mark.timeout(600)
def test_backward_long_context_prefix():
    """The long-context workload in full (T = 32768, H_q = 32, H_kv = 8,
    d = 128, vector gate, 1% of key rows x8; workspace 680 MB) with dO zero
    from token T0 = 2048 on. By causality only the first T0 outputs carry
    loss, so the gradients of the first T0 tokens are those of the T0-token
    prefix problem and every gradient from T0 on is zero. The prefix problem
    is run through the same call and checked against the float64 reverse
    pass; the long run must agree with it on the first T0 tokens (same chunk
    records and scans there) and be exactly zero after."""
    from synth import config_prefill_inputs
    T0 = 2048
    x = config_prefill_inputs("prefill_8b_b1_t32768_d128_outliers")
    T = x["q"].shape[1]
    dO = grad_output(x["q"].shape, "bf16", seed=31)
    dO[:, T0:] = 0.0
    assert gla.liger_attn_prefill_backward_workspace_size(1, T, 32, 8, 128) > 600e6
    say(f"[bwd] long context T={T}: GPU")
    got = _run(x, dO, 1, 64, 0.5)
    xp = {n: np.ascontiguousarray(x[n][:, :T0]) for n in ("q", "k", "v")}
    dOp = np.ascontiguousarray(dO[:, :T0])
    say(f"[bwd] prefix T0={T0}: GPU")
    pre = _run(xp, dOp, 1, 64, 0.5)
    say(f"[bwd] prefix T0={T0}: oracle")
    ref = oracle.prefill_backward(xp["q"], xp["k"], xp["v"], dOp, 1, 64, 0.5)
    _check(pre, ref, "bwd long-context prefix")
    for name, a, p in zip(("dq", "dk", "dv"), got, pre):
        assert np.all(np.isfinite(a)), f"{name} has non-finite entries"
        scale = max(float(np.max(np.abs(p))), 1e-30)
        err = float(np.max(np.abs(a[:, :T0] - p))) / scale
        assert err <= 1e-6, (name, err)
        assert not np.any(a[:, T0:]), f"{name}: non-zero gradient after T0"
