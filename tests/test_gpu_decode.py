"""GPU parity of the decode step (and ring set-up) against the float64 oracle.

Checks: outputs at every step, the fp32 state, the ring contents bit for
bit, pos and the arrival counters; the state layout with structured inputs;
resume from a host snapshot; the 64-sequence, 1024-step Llama-3-8B workload.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrent_amd as gla
import oracle
from liger_testutil import DEV, TORCH_DT, abs_inf, rel_inf, say, to_dev, to_np
from synth import CONFIGS, GATE_MODES, decode_initial, decode_step_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _bars(dtype, o_gpu, o_ref, tag):
    if dtype == "f32":
        assert rel_inf(o_gpu, o_ref) <= 1e-4, (tag, rel_inf(o_gpu, o_ref))
    else:
        assert abs_inf(o_gpu, o_ref) <= 2e-2, (tag, abs_inf(o_gpu, o_ref))


def _ring_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def _np_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    return _ring_bits(to_dev(a, dtype))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("n_rep,window,T0", [(1, 64, 70), (4, 17, 3), (8, 64, 1), (2, 1, 5)])
def test_prefill_then_decode_matches_oracle(dtype, d, gate, n_rep, window, T0):
    n_steps = 12
    N, H_kv = 3, 2
    H_q = H_kv * n_rep
    tag = f"decode {dtype} d={d} gate={gate} n_rep={n_rep} w={window} T0={T0}"
    say(f"[decode] {tag}")
    x = prefill_inputs(B=N, T=T0 + n_steps, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, seed=T0 + 31 * n_rep)
    o_full, S_full = oracle.prefill(x["q"], x["k"], x["v"], gate, window, 0.5)
    # the state after the prompt comes from the oracle (fp32 path parity of
    # prefill is tested separately; d=128 fp32 has no prefill kernel)
    _, S0 = oracle.prefill(x["q"][:, :T0], x["k"][:, :T0], x["v"][:, :T0], gate, window, 0.5)
    S = torch.from_numpy(S0.astype(np.float32)).to(DEV)
    ring = gla.KVRing.empty(N, H_kv, window, d, TORCH_DT[dtype], DEV)
    gla.liger_kv_ring_fill(to_dev(x["k"][:, :T0], dtype), to_dev(x["v"][:, :T0], dtype), ring)
    for i in range(n_steps):
        t = T0 + i
        o = gla.liger_attn_decode_step(to_dev(x["q"][:, t], dtype), to_dev(x["k"][:, t], dtype),
                                       to_dev(x["v"][:, t], dtype), S, ring, gate, 0.5)
        torch.cuda.synchronize()
        _bars(dtype, to_np(o), o_full[:, t], f"{tag} step {i}")
    assert rel_inf(to_np(S), S_full) <= 1e-5, rel_inf(to_np(S), S_full)
    rk, rv, pos = oracle.ring_fill(x["k"], x["v"], window)
    assert np.array_equal(_ring_bits(ring.k), _np_bits(rk, dtype))
    assert np.array_equal(_ring_bits(ring.v), _np_bits(rv, dtype))
    assert np.array_equal(ring.pos.cpu().numpy(), pos)
    assert int(ring.sync.abs().sum()) == 0


@pytest.mark.parametrize("gate", [0, 1])
def test_gpu_prefill_hands_over_to_decode(gate):
    """GPU prefill state + ring fill + GPU decode continues the sequence."""
    N, H_kv, n_rep, d, T0, n = 2, 2, 4, 128, 300, 20
    say(f"[decode] prefill hand-over gate={gate}")
    x = prefill_inputs(B=N, T=T0 + n, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=77)
    o_full, S_full = oracle.prefill(x["q"], x["k"], x["v"], gate, 64, 0.5)
    _, S = gla.liger_attn_prefill(to_dev(x["q"][:, :T0], "bf16"), to_dev(x["k"][:, :T0], "bf16"),
                                  to_dev(x["v"][:, :T0], "bf16"), gate, 64, 0.5)
    ring = gla.KVRing.empty(N, H_kv, 64, d, torch.bfloat16, DEV)
    gla.liger_kv_ring_fill(to_dev(x["k"][:, :T0], "bf16"), to_dev(x["v"][:, :T0], "bf16"), ring)
    for i in range(n):
        t = T0 + i
        o = gla.liger_attn_decode_step(to_dev(x["q"][:, t], "bf16"), to_dev(x["k"][:, t], "bf16"),
                                       to_dev(x["v"][:, t], "bf16"), S, ring, gate, 0.5)
        torch.cuda.synchronize()
        assert abs_inf(to_np(o), o_full[:, t]) <= 2e-2
    assert rel_inf(to_np(S), S_full) <= 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", [0, 1])
def test_state_layout_bit_exact(dtype, gate):
    """S0[n,h,i,j] encodes its own index; with k = 0 (gate 1/2, phi(k) = 1/d)
    and v = 0 one step must give exactly S0 / 2 in every element."""
    N, H_kv, n_rep, d, w = 2, 3, 2, 128, 8
    say(f"[decode] state layout {dtype} gate={gate}")
    i = np.arange(d, dtype=np.float32)
    S0 = (i[:, None] + i[None, :] / 256.0)[None, None] + \
        (np.arange(N, dtype=np.float32)[:, None, None, None] * 1000 + np.arange(H_kv, dtype=np.float32)[None, :, None, None] * 100)
    S = torch.from_numpy(np.ascontiguousarray(S0, np.float32)).to(DEV)
    ring = gla.KVRing.empty(N, H_kv, w, d, TORCH_DT[dtype], DEV)
    ring.pos.fill_(5)
    q = torch.randn(N, H_kv * n_rep, d, device=DEV).to(TORCH_DT[dtype])
    z = torch.zeros(N, H_kv, d, device=DEV, dtype=TORCH_DT[dtype])
    gla.liger_attn_decode_step(q, z, z, S, ring, gate, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), (S0 * np.float32(0.5)).astype(np.float32))
    assert np.array_equal(ring.pos.cpu().numpy(), [6, 6])


def test_resume_from_host_snapshot():
    N, H_kv, n_rep, d, w = 4, 2, 4, 128, 64
    say("[decode] resume from snapshot")
    init = decode_initial(N=N, H_kv=H_kv, d=d, window=w, dtype="bf16", seed=9, pos0=100)
    steps = [decode_step_inputs(N=N, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=9, step=s)
             for s in range(16)]

    def fresh():
        ring = gla.KVRing(to_dev(init["ring_k"], "bf16"), to_dev(init["ring_v"], "bf16"),
                          torch.from_numpy(init["pos"]).to(DEV), torch.zeros(N, dtype=torch.int32, device=DEV), w)
        return torch.from_numpy(init["S"]).to(DEV), ring

    def step(S, ring, s):
        x = steps[s]
        return gla.liger_attn_decode_step(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                                          S, ring, 1, 0.5)

    S, ring = fresh()
    ref = [step(S, ring, s).clone() for s in range(16)]
    S2, ring2 = fresh()
    for s in range(8):
        step(S2, ring2, s)
    torch.cuda.synchronize()
    snap = [t.cpu().clone() for t in (S2, ring2.k, ring2.v, ring2.pos, ring2.sync)]
    S3 = snap[0].to(DEV)
    ring3 = gla.KVRing(snap[1].to(DEV), snap[2].to(DEV), snap[3].to(DEV), snap[4].to(DEV), w)
    for s in range(8, 16):
        o = step(S3, ring3, s)
        assert torch.equal(o, ref[s])
    assert torch.equal(S3, S) and torch.equal(ring3.k, ring.k) and torch.equal(ring3.pos, ring.pos)


def test_config_decode_8b_full():
    """64 sequences x 1024 steps at Llama-3-8B geometry (all sequences on the
    GPU; the oracle follows four of them, since sequences are independent)."""
    name = "decode_8b_n64_d128"
    cfg = CONFIGS[name]
    N, H_q, H_kv, d, w = cfg["N"], cfg["H_q"], cfg["H_kv"], cfg["d"], cfg["window"]
    gate = GATE_MODES[cfg["gate"]]
    follow = np.array([0, 17, 42, 63])
    say(f"[decode] {name} steps={cfg['steps']} following sequences {follow.tolist()}")
    init = decode_initial(**cfg)
    S = torch.from_numpy(init["S"]).to(DEV)
    ring = gla.KVRing(to_dev(init["ring_k"], "bf16"), to_dev(init["ring_v"], "bf16"),
                      torch.from_numpy(init["pos"]).to(DEV), torch.zeros(N, dtype=torch.int32, device=DEV), w)
    S_ref = init["S"][follow].astype(np.float64)
    rk_ref, rv_ref, pos_ref = init["ring_k"][follow], init["ring_v"][follow], init["pos"][follow]
    worst = 0.0
    for s in range(cfg["steps"]):
        x = decode_step_inputs(step=s, **cfg)
        o = gla.liger_attn_decode_step(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
                                       S, ring, gate, cfg["alpha"])
        o_ref, S_ref, rk_ref, rv_ref, pos_ref = oracle.decode_step(
            x["q"][follow], x["k"][follow], x["v"][follow], S_ref, rk_ref, rv_ref, pos_ref, gate, cfg["alpha"])
        err = abs_inf(to_np(o)[follow], o_ref)
        worst = max(worst, err)
        assert err <= 2e-2, (s, err)
        if s % 256 == 0:
            say(f"  step {s}: max|o - ref| = {err:.3e}")
    say(f"  worst max|o - ref| over all steps: {worst:.3e}")
    assert rel_inf(to_np(S)[follow], S_ref) <= 1e-4
    assert np.array_equal(_ring_bits(ring.k)[follow], _np_bits(rk_ref, "bf16"))
    assert np.array_equal(_ring_bits(ring.v)[follow], _np_bits(rv_ref, "bf16"))
    assert np.array_equal(ring.pos.cpu().numpy(), np.full(N, cfg["pos0"] + cfg["steps"]))
    assert int(ring.sync.abs().sum()) == 0
