"""GPU parity of the hybrid's full causal softmax attention layer against the
float64 oracle (bf16 inputs, max |gpu - ref| <= 2e-2 on the unit-scale
output, the bar of the bf16 path).

Small shapes compare every output; the 8B shape (T = 8192, 32 query heads,
8 key/value heads, d = 128) compares sampled query rows, each recomputed in
float64 from its full causal prefix.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrent_amd as gla
import oracle
from liger_testutil import DEV, abs_inf, say, to_dev, to_np
from synth import config_prefill_inputs, prefill_inputs

pytestmark = pytest.mark.gpu

BAR = 2e-2


def _run(x):
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    gla.liger_attn_full_causal(q, k, v, o=o)
    torch.cuda.synchronize()
    return to_np(o)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8])
@pytest.mark.parametrize("B,T", [(1, 1), (2, 37), (1, 64), (2, 130), (1, 300)])
def test_full_matches_oracle(d, n_rep, B, T):
    H_kv = 2 if n_rep < 8 else 1
    say(f"[full] d={d} n_rep={n_rep} B={B} T={T}")
    x = prefill_inputs(B=B, T=T, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=1000 + T + 7 * n_rep + d)
    ref = oracle.full_attention(x["q"], x["k"], x["v"])
    err = abs_inf(_run(x), ref)
    assert err <= BAR, (d, n_rep, B, T, err)


def test_full_spiky_scores():
    """Queries scaled x8: near one-hot rows stress the running maximum."""
    x = prefill_inputs(B=1, T=200, H_q=8, H_kv=2, d=128, dtype="bf16", seed=5)
    x["q"] = x["q"] * 8.0  # powers of two keep the values bf16-exact
    ref = oracle.full_attention(x["q"], x["k"], x["v"])
    err = abs_inf(_run(x), ref)
    assert err <= BAR, err


def test_full_8b_shape_sampled_rows():
    """T = 8192, H_q = 32, H_kv = 8, d = 128 (the 8B prefill inputs)."""
    x = config_prefill_inputs("prefill_8b_b1_t8192_d128")
    say("[full] 8B shape")
    o = _run(x)
    q, k, v = (np.asarray(x[n], np.float64) for n in ("q", "k", "v"))
    T, H_q, d = q.shape[1], q.shape[2], q.shape[3]
    n_rep = H_q // k.shape[2]
    rows = [0, 1, 63, 64, 65, 1000, 4095, 4096, 8000, T - 1]
    worst = 0.0
    for t in rows:
        for h in (0, 5, 17, 31):
            kh, vh = k[0, :t + 1, h // n_rep], v[0, :t + 1, h // n_rep]
            s = kh @ q[0, t, h] / np.sqrt(d)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ vh
            worst = max(worst, float(np.max(np.abs(o[0, t, h] - ref))))
    assert worst <= BAR, worst
    assert np.isfinite(o).all()
