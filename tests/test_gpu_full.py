"""GPU parity of the hybrid's full causal softmax attention layer against the
float64 oracle (bf16 inputs).

Bars: small shapes compare every output, max |gpu - ref| <= 2e-2 (the bf16
path's bar on unit-scale outputs). Long sequences have small outputs late in
the sequence (|o| ~ 1/sqrt(t)), so there every checked row must also satisfy
a relative bar of its own: max_c |gpu - ref| <= 2e-2 * max_c |ref| per
(query row, head). The 8B shape (T = 8192, 32 query heads, 8 key/value
heads, d = 128) checks one row in every 64-query block, for all 32 heads,
against oracle.full_attention_rows.
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
ROW_REL_BAR = 2e-2


def _run(x):
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    gla.liger_attn_full_causal(q, k, v, o=o)
    torch.cuda.synchronize()
    return to_np(o)


def _row_rel(o_rows, ref_rows):
    """Worst per-(row, head) error relative to that row's largest |ref|."""
    err = np.max(np.abs(o_rows - ref_rows), axis=-1)
    scale = np.max(np.abs(ref_rows), axis=-1)
    return float(np.max(err / scale))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8])
@pytest.mark.parametrize("B,T", [(1, 1), (2, 37), (1, 64), (2, 130), (1, 300)])
def test_full_matches_oracle(d, n_rep, B, T):
    H_kv = 2 if n_rep < 8 else 1
    say(f"[full] d={d} n_rep={n_rep} B={B} T={T}")
    x = prefill_inputs(B=B, T=T, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=1000 + T + 7 * n_rep + d)
    ref = oracle.full_attention(x["q"], x["k"], x["v"])
    o = _run(x)
    err = abs_inf(o, ref)
    assert err <= BAR, (d, n_rep, B, T, err)
    rel = _row_rel(o, ref)
    assert rel <= ROW_REL_BAR, (d, n_rep, B, T, rel)


# (B, H_q, H_kv): B * (query-head groups of up to 4 heads) is a multiple of 8,
# the case whose workgroups are ordered so that each group stays on one XCD
@pytest.mark.parametrize("B,H_q,H_kv", [(1, 32, 8), (4, 8, 2), (2, 16, 8)])
@pytest.mark.parametrize("d", [64, 128])
def test_full_xcd_grouped_order_matches_oracle(B, H_q, H_kv, d):
    T = 300
    say(f"[full] XCD-ordered groups B={B} H_q={H_q} H_kv={H_kv} d={d} T={T}")
    x = prefill_inputs(B=B, T=T, H_q=H_q, H_kv=H_kv, d=d, dtype="bf16", seed=77 + B + H_q + d)
    ref = oracle.full_attention(x["q"], x["k"], x["v"])
    o = _run(x)
    err = abs_inf(o, ref)
    rel = _row_rel(o, ref)
    say(f"  max abs {err:.3e}, worst row-relative {rel:.3e}")
    assert err <= BAR and rel <= ROW_REL_BAR, (err, rel)


def test_full_spiky_scores():
    """Queries scaled x8: near one-hot rows stress the running maximum."""
    x = prefill_inputs(B=1, T=200, H_q=8, H_kv=2, d=128, dtype="bf16", seed=5)
    x["q"] = x["q"] * 8.0  # powers of two keep the values bf16-exact
    ref = oracle.full_attention(x["q"], x["k"], x["v"])
    o = _run(x)
    err = abs_inf(o, ref)
    assert err <= BAR, err
    assert _row_rel(o, ref) <= ROW_REL_BAR


@pytest.mark.timeout(300)
def test_full_8b_shape_every_query_block():
    """T = 8192, H_q = 32, H_kv = 8, d = 128 (the 8B prefill inputs): one row
    per 64-query block (offset varying with the block, the first and last
    rows included), all 32 heads, against oracle.full_attention_rows."""
    x = config_prefill_inputs("prefill_8b_b1_t8192_d128")
    say("[full] 8B shape, one row per query block, all heads")
    o = _run(x)
    assert np.isfinite(o).all()
    T = o.shape[1]
    rows = sorted({64 * blk + (37 * blk + 11) % 64 for blk in range(T // 64)} | {0, 63, 64, T - 1})
    ref = oracle.full_attention_rows(x["q"], x["k"], x["v"], rows)
    got = o[:, rows]
    err = abs_inf(got, ref)
    rel = _row_rel(got, ref)
    say(f"  {len(rows)} rows x 32 heads: max abs {err:.3e}, worst row-relative {rel:.3e}")
    assert err <= BAR, err
    assert rel <= ROW_REL_BAR, rel
