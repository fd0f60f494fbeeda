"""The allocation-free prefill entry point (liger_attn_prefill_noalloc).

It must give the same outputs as liger_attn_prefill (the same kernels, the
workspace taken from the library's static scratch instead of a caller
buffer) on consecutive calls that reuse the scratch, the second one
smaller, and both within the oracle's parity bars. Called through the C ABI.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrent_amd as gla
import oracle
from liger_testutil import DEV, check_prefill, say, to_dev, to_np
from synth import config_prefill_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _both(x, dtype, gate, window, alpha):
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    o_ref, S_ref = gla.liger_attn_prefill(q, k, v, gate, window, alpha)
    o = torch.full_like(q, float("nan"))
    S_T = torch.full((B, H_kv, d, d), float("nan"), dtype=torch.float32, device=DEV)
    gla.liger_attn_prefill_noalloc(q, k, v, gate, window, alpha, o=o, S_T=S_T)
    torch.cuda.synchronize()
    return o, S_T, o_ref, S_ref


@pytest.mark.timeout(300)
def test_noalloc_matches_prefill_on_consecutive_calls():
    """First the 8B workload (T = 8192, 32 query heads, 8 key/value heads,
    d = 128: 31.6 MiB of the 32 MiB scratch), then a smaller, ragged vector-gate
    case, then fp32 cases at d = 64 and d = 128: each bit-identical to liger_attn_prefill and
    within the parity bars against the oracle."""
    assert gla.liger_attn_prefill_noalloc_max_workspace() == 32 << 20
    say("[noalloc] 8B workload")
    x = config_prefill_inputs("prefill_8b_b1_t8192_d128")
    need = gla.liger_attn_prefill_workspace_size(1, 8192, 32, 8, 128, gla.LIGER_BF16)
    assert 30 << 20 < need <= 32 << 20, need
    o, S, o_ref, S_ref = _both(x, "bf16", 0, 64, 0.5)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(S, S_ref)
    rows = [0, 63, 64, 4095, 8191]
    ref_o, ref_S = oracle.prefill(x["q"], x["k"], x["v"], 0, 64, 0.5)
    check_prefill("bf16", to_np(o)[:, rows], ref_o[:, rows], to_np(S), ref_S, tag="noalloc 8B")

    for dtype, d, gate, (B, T, H_q, H_kv), window, alpha in [
            ("bf16", 128, 1, (2, 300, 8, 2), 64, 0.5),
            ("f32", 64, 0, (1, 200, 4, 1), 17, 1.0),
            ("f32", 128, 1, (1, 330, 8, 2), 64, 0.5)]:
        say(f"[noalloc] {dtype} d={d} gate={gate} B={B} T={T} H_q={H_q} H_kv={H_kv} w={window} alpha={alpha}")
        x = prefill_inputs(B=B, T=T, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, seed=T + d)
        o, S, o_ref, S_ref = _both(x, dtype, gate, window, alpha)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
        ref_o, ref_S, ref_grm, _ = oracle.prefill(x["q"], x["k"], x["v"], gate, window, alpha, return_parts=True)
        if alpha == 1.0:
            check_prefill(dtype, to_np(o), ref_o, to_np(S), ref_S, o1_gpu=to_np(o), o1_ref=ref_grm,
                          tag="noalloc small")
        else:
            check_prefill(dtype, to_np(o), ref_o, to_np(S), ref_S, tag="noalloc small")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the scratch is refused before any launch."""
    need = gla.liger_attn_prefill_workspace_size(65, 64, 32, 8, 128, gla.LIGER_BF16)
    assert need > 32 << 20
    q = torch.zeros(65, 64, 32, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(65, 64, 8, 128, dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    S = torch.empty(65, 8, 128, 128, dtype=torch.float32, device=DEV)
    with pytest.raises(gla.LigerError) as e:
        gla.liger_attn_prefill_noalloc(q, k, k, 0, 64, 0.5, o=o, S_T=S)
    assert e.value.status == gla.LIGER_E_WORKSPACE
