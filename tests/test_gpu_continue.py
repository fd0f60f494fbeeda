"""GPU parity of the prefill continuation against the float64 oracle.

A continuation of T2 tokens after T1 consumed ones must equal one prefill
of the T1 + T2 tokens restricted to the new ones (the oracle's
prefill_continue is pinned to that on the CPU): outputs, the final state,
the ring contents bit for bit, pos and the arrival counters. The state and
ring entering the continuation come from the oracle (so the continuation is
tested alone) or from the GPU prefill and ring fill (the hand-over).
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrent_amd as gla
import oracle
from liger_testutil import DEV, TORCH_DT, check_prefill, say, to_dev, to_np
from synth import config_prefill_inputs, prefill_inputs, round_to_bf16

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _ring_from(rk, rv, pos, window, dtype):
    B, H_kv, _, d = rk.shape
    return gla.KVRing(to_dev(rk, dtype), to_dev(rv, dtype), torch.from_numpy(np.asarray(pos, np.int64)).to(DEV),
                      torch.zeros(B, dtype=torch.int32, device=DEV), window)


def _check_ring(ring, rk, rv, pos, dtype, tag):
    assert np.array_equal(_bits(ring.k), _bits(to_dev(rk, dtype))), tag
    assert np.array_equal(_bits(ring.v), _bits(to_dev(rv, dtype))), tag
    assert np.array_equal(ring.pos.cpu().numpy(), pos), (tag, ring.pos.cpu().numpy(), pos)
    assert int(ring.sync.abs().sum()) == 0, tag


def _run(dtype, d, gate, n_rep, window, T1, T2, alpha=0.5, B=2, H_kv=2, seed=0):
    H_q = H_kv * n_rep
    tag = f"continue {dtype} d={d} gate={gate} n_rep={n_rep} w={window} T1={T1} T2={T2}"
    say(f"[continue] {tag}")
    x = prefill_inputs(B=B, T=T1 + T2, H_q=H_q, H_kv=H_kv, d=d, dtype=dtype, seed=seed or (7 * T1 + T2))
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full, o1_full, _ = oracle.prefill(q, k, v, gate, window, alpha, return_parts=True)
    if T1 > 0:
        _, S0 = oracle.prefill(q[:, :T1], k[:, :T1], v[:, :T1], gate, window, alpha)
    else:
        S0 = np.zeros((B, H_kv, d, d))
    rk, rv, pos = oracle.ring_fill(k[:, :T1], v[:, :T1], window)
    ring = _ring_from(rk, rv, pos, window, dtype)
    S0_dev = torch.from_numpy(S0.astype(np.float32)).to(DEV)
    qd, kd, vd = (to_dev(a[:, T1:], dtype) for a in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    S_T = torch.full_like(S0_dev, float("nan"))
    gla.liger_attn_prefill_continue(qd, kd, vd, S0_dev, ring, gate, alpha, o=o, S_T=S_T)
    torch.cuda.synchronize()
    if alpha == 1.0:
        # the recurrent output alone: its own relative bar (the window output
        # is ~25x larger and would hide a wrong recurrence under the mixed bar)
        check_prefill(dtype, to_np(o), o1_full[:, T1:], to_np(S_T), S_full, o1_gpu=to_np(o),
                      o1_ref=o1_full[:, T1:], tag=tag)
    else:
        check_prefill(dtype, to_np(o), o_full[:, T1:], to_np(S_T), S_full, tag=tag)
    assert np.array_equal(to_np(S0_dev), S0.astype(np.float32)), f"{tag}: S0 modified"
    rk_ref, rv_ref, pos_ref = oracle.ring_fill(k, v, window)
    _check_ring(ring, rk_ref, rv_ref, pos_ref, dtype, tag)
    return x


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("n_rep,window,T1,T2", [
    (1, 64, 0, 100),     # from a zero state and an empty ring: a plain prefill
    (4, 64, 1, 63),      # one token of history
    (4, 64, 30, 65),     # fewer than 64 tokens of history
    (1, 64, 64, 64),     # exactly one chunk of history
    (4, 17, 100, 1),     # one new token, small window
    (2, 64, 200, 130),   # several chunks on both sides
    (4, 1, 50, 70),      # window 1
])
def test_continue_matches_oracle(dtype, d, gate, n_rep, window, T1, T2):
    _run(dtype, d, gate, n_rep, window, T1, T2)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("alpha", [0.0, 1.0])
@pytest.mark.parametrize("n_rep,window,T1,T2", [
    (4, 64, 30, 65),     # fewer than 64 tokens of history, a ragged chunk
    (2, 64, 200, 130),   # several chunks on both sides
    (2, 1, 5, 70),       # window 1
])
def test_continue_mixers_alone(dtype, d, gate, alpha, n_rep, window, T1, T2):
    """alpha = 1 (recurrent output alone, relative bar) and alpha = 0 (window alone)."""
    _run(dtype, d, gate, n_rep, window, T1, T2, alpha=alpha)


@pytest.mark.parametrize("alpha", [0.0, 1.0])
def test_continue_many_segments_mixers_alone(alpha):
    """A long continuation (several segments, carried state in the carry scan)
    with each mixer alone."""
    _run("bf16", 128, 1, 4, 64, 150, 2100, B=1, H_kv=2, alpha=alpha)


@pytest.mark.parametrize("gate", [0, 1])
def test_continue_many_segments(gate):
    """Long continuation: several segments, so the carried state enters the carry scan."""
    _run("bf16", 128, gate, 4, 64, 150, 2100, B=1, H_kv=2)


def test_continue_per_sequence_positions():
    """Sequences with different histories (pos differs per sequence)."""
    dtype, d, gate, window, alpha, H_kv, n_rep, T2 = "bf16", 128, 1, 64, 0.5, 2, 4, 90
    T1s = [5, 170]
    B = len(T1s)
    say("[continue] per-sequence positions")
    xs = [prefill_inputs(B=1, T=t1 + T2, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype=dtype, seed=40 + i)
          for i, t1 in enumerate(T1s)]
    S0 = np.zeros((B, H_kv, d, d))
    rk = np.zeros((B, H_kv, window, d), np.float32)
    rv = np.zeros_like(rk)
    pos = np.zeros(B, np.int64)
    o_ref, S_ref = [], []
    for i, (x, t1) in enumerate(zip(xs, T1s)):
        q, k, v = x["q"], x["k"], x["v"]
        of, sf = oracle.prefill(q, k, v, gate, window, alpha)
        o_ref.append(of[0, t1:])
        S_ref.append(sf[0])
        _, s1 = oracle.prefill(q[:, :t1], k[:, :t1], v[:, :t1], gate, window, alpha)
        S0[i] = s1[0]
        a, bb, p = oracle.ring_fill(k[:, :t1], v[:, :t1], window)
        rk[i], rv[i], pos[i] = a[0], bb[0], p[0]
    ring = _ring_from(rk, rv, pos, window, dtype)
    new = {n: np.concatenate([x[n][:, t1:] for x, t1 in zip(xs, T1s)]) for n in ("q", "k", "v")}
    qd, kd, vd = (to_dev(new[n], dtype) for n in ("q", "k", "v"))
    o, S_T = gla.liger_attn_prefill_continue(qd, kd, vd, torch.from_numpy(S0.astype(np.float32)).to(DEV), ring,
                                             gate, alpha)
    torch.cuda.synchronize()
    check_prefill(dtype, to_np(o), np.stack(o_ref), to_np(S_T), np.stack(S_ref), tag="per-sequence pos")
    for i, (x, t1) in enumerate(zip(xs, T1s)):
        a, bb, p = oracle.ring_fill(x["k"], x["v"], window)
        assert np.array_equal(_bits(ring.k[i]), _bits(to_dev(a[0], dtype)))
        assert np.array_equal(_bits(ring.v[i]), _bits(to_dev(bb[0], dtype)))
        assert int(ring.pos[i]) == int(p[0])


@pytest.mark.parametrize("gate", [0, 1])
def test_gpu_prefill_hands_over_to_continuation(gate):
    """GPU prefill of T1 tokens, GPU ring fill, then a GPU continuation."""
    dtype, d, window, alpha, T1, T2 = "bf16", 128, 64, 0.5, 330, 200
    x = prefill_inputs(B=2, T=T1 + T2, H_q=8, H_kv=2, d=d, dtype=dtype, seed=77 + gate)
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full = oracle.prefill(q, k, v, gate, window, alpha)
    say(f"[continue] hand-over gate={gate}")
    q1, k1, v1 = (to_dev(a[:, :T1], dtype) for a in (q, k, v))
    _, S1 = gla.liger_attn_prefill(q1, k1, v1, gate, window, alpha)
    ring = gla.KVRing.empty(2, 2, window, d, TORCH_DT[dtype], DEV)
    gla.liger_kv_ring_fill(k1, v1, ring)
    q2, k2, v2 = (to_dev(a[:, T1:], dtype) for a in (q, k, v))
    o2, S2 = gla.liger_attn_prefill_continue(q2, k2, v2, S1, ring, gate, alpha)
    torch.cuda.synchronize()
    check_prefill(dtype, to_np(o2), o_full[:, T1:], to_np(S2), S_full, tag="hand-over")
    rk, rv, pos = oracle.ring_fill(k, v, window)
    _check_ring(ring, rk, rv, pos, dtype, "hand-over")


@pytest.mark.parametrize("gate", [0, 1])
def test_slow_decay_hands_over_to_continuation(gate):
    """Keys shifted by +6 (gates ~0.9975, phi(k) unchanged): the state the GPU
    prefill hands over still weighs on every continued token. alpha = 1: the
    recurrent output alone, held to its relative bar."""
    dtype, d, window, alpha, T1, T2 = "bf16", 128, 64, 1.0, 330, 200
    x = prefill_inputs(B=2, T=T1 + T2, H_q=8, H_kv=2, d=d, dtype=dtype, seed=79 + gate)
    x["k"] = round_to_bf16(x["k"] + 6.0)
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full = oracle.prefill(q, k, v, gate, window, alpha)
    say(f"[continue] slow-decay hand-over gate={gate}")
    q1, k1, v1 = (to_dev(a[:, :T1], dtype) for a in (q, k, v))
    _, S1 = gla.liger_attn_prefill(q1, k1, v1, gate, window, alpha)
    ring = gla.KVRing.empty(2, 2, window, d, TORCH_DT[dtype], DEV)
    gla.liger_kv_ring_fill(k1, v1, ring)
    q2, k2, v2 = (to_dev(a[:, T1:], dtype) for a in (q, k, v))
    o2, S2 = gla.liger_attn_prefill_continue(q2, k2, v2, S1, ring, gate, alpha)
    torch.cuda.synchronize()
    check_prefill(dtype, to_np(o2), o_full[:, T1:], to_np(S2), S_full, to_np(o2), o_full[:, T1:],
                  tag="slow-decay hand-over")


@pytest.mark.timeout(300)
def test_continuation_8b_shape_full():
    """The 8B prefill workload (T = 8192, H_q = 32, H_kv = 8, d = 128, scalar
    gate) split at a ragged boundary: GPU prefill of the first 4000 tokens,
    GPU ring fill, GPU continuation over the other 4192; outputs, the final
    state and the ring against one oracle prefill of all 8192 tokens."""
    dtype, T1 = "bf16", 4000
    say("[continue] 8B shape, 4000 + 4192")
    x = config_prefill_inputs("prefill_8b_b1_t8192_d128")
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full = oracle.prefill(q, k, v, 0, 64, 0.5)
    q1, k1, v1 = (to_dev(a[:, :T1], dtype) for a in (q, k, v))
    _, S1 = gla.liger_attn_prefill(q1, k1, v1, 0, 64, 0.5)
    ring = gla.KVRing.empty(1, 8, 64, 128, TORCH_DT[dtype], DEV)
    gla.liger_kv_ring_fill(k1, v1, ring)
    q2, k2, v2 = (to_dev(a[:, T1:], dtype) for a in (q, k, v))
    o2, S2 = gla.liger_attn_prefill_continue(q2, k2, v2, S1, ring, 0, 0.5)
    torch.cuda.synchronize()
    check_prefill(dtype, to_np(o2), o_full[:, T1:], to_np(S2), S_full, tag="continuation 8B shape")
    rk, rv, pos = oracle.ring_fill(k, v, 64)
    _check_ring(ring, rk, rv, pos, dtype, "continuation 8B shape")
