"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test states what it pins and which plausible mistake it would catch.
None of these recompute the oracle's own formula: they use a different form
of the same definition (parallel vs recurrent), a library routine, a closed
form derived by hand, or an invariant of the mathematics.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from synth import prefill_inputs, round_to_bf16

SEEDS = range(20)


# ---------------------------------------------------------------- helpers
# Independent implementations used only by the pins.

def _softmax_lib(x):
    return sps.softmax(np.asarray(x, np.float64), axis=-1)


def _gate_indep(k, mode):
    """Gate via prefix sums (different route from the oracle's slicing)."""
    k = np.asarray(k, np.float64)
    d = k.shape[-1]
    if mode == oracle.SCALAR_MEAN:
        s = np.sum(k, axis=-1, keepdims=True) / d
        return np.broadcast_to(sps.expit(s), k.shape)
    cs = np.concatenate([np.zeros(k.shape[:-1] + (1,)), np.cumsum(k, axis=-1)], axis=-1)
    out = np.empty_like(k)
    for c in range(d):
        lo, hi = max(0, c - 1), min(d, c + 3)
        out[..., c] = (cs[..., hi] - cs[..., lo]) / (hi - lo)
    return sps.expit(out)


def _brute_force(q, k, v, mode, window, alpha):
    """O(T^2) parallel form with explicit products of the per-token gates.

    o_grm[t] = sum_{j<=t} sum_i phi_q[t,i] phi_k[j,i] (prod_{s=j+1..t} g_s[i]) v_j
    S_T      = sum_j diag(prod_{s=j+1..T-1} g_s) phi_k[j]^T v_j
    o_swa[t] = sum over keys j in [t-window+1, t] of softmax_j(q_t.k_j/sqrt d) v_j
    """
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    n_rep = H_q // H_kv
    g = _gate_indep(k, mode)                       # [B, T, H_kv, d]
    pq, pk = _softmax_lib(q), _softmax_lib(k)
    o = np.zeros_like(q)
    o_grm = np.zeros_like(q)
    S_T = np.zeros((B, H_kv, d, d))
    for b in range(B):
        for h in range(H_q):
            hk = h // n_rep
            for t in range(T):
                acc = np.zeros(d)
                for j in range(t + 1):
                    dec = np.prod(g[b, j + 1:t + 1, hk], axis=0)  # empty product = 1
                    acc += np.sum(pq[b, t, h] * pk[b, j, hk] * dec) * v[b, j, hk]
                o_grm[b, t, h] = acc
                lo = max(0, t - window + 1)
                logits = np.array([q[b, t, h] @ k[b, j, hk] for j in range(lo, t + 1)]) / math.sqrt(d)
                p = np.exp(logits - logits.max())
                p /= p.sum()
                swa = sum(p[i] * v[b, lo + i, hk] for i in range(len(p)))
                o[b, t, h] = alpha * acc + (1 - alpha) * swa
        for hk in range(H_kv):
            for j in range(T):
                dec = np.prod(g[b, j + 1:T, hk], axis=0)
                S_T[b, hk] += (dec * pk[b, j, hk])[:, None] * v[b, j, hk][None, :]
    return o, S_T, o_grm


def _close(a, b, rtol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b))))
    return float(np.max(np.abs(a - b))) <= rtol * scale


# ------------------------------------------------------------------- pins

@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
@pytest.mark.parametrize("n_rep", [1, 2, 4])
@pytest.mark.parametrize("seed", SEEDS)
def test_recurrence_equals_bruteforce_parallel_form(mode, n_rep, seed):
    """Pin 1: recurrence vs O(T^2) parallel form with the explicit decay product.

    Catches: a gate on the wrong axis of S, a transposed state, an exclusive
    diagonal (o_t using S_{t-1}), an off-by-one window edge, gates taken from
    phi(k) instead of raw k, a wrong GQA head map.
    """
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 21))
    d = int(rng.choice([4, 6, 8]))
    H_kv = int(rng.integers(1, 3))
    window = int(rng.integers(1, T + 3))
    alpha = float(rng.uniform(0.0, 1.0))
    q = rng.standard_normal((1, T, H_kv * n_rep, d)) * 1.5
    k = rng.standard_normal((1, T, H_kv, d)) * 1.5
    v = rng.standard_normal((1, T, H_kv, d))
    o, S, _, _ = oracle.prefill(q, k, v, mode, window, alpha, return_parts=True)
    o_bf, S_bf, _ = _brute_force(q, k, v, mode, window, alpha)
    assert _close(o, o_bf) and _close(S, S_bf)


def test_pool_vector_hand_example():
    """Pin: kernel-4 'same' average with an in-range divisor, worked by hand.

    k = [4, 0, 8, 0, 0, 12] (d = 6); windows [c-1, c+2] clipped to [0, 5]:
      c=0 {0,1,2}: 12/3 = 4     c=3 {2,3,4,5}: 20/4 = 5
      c=1 {0..3}:  12/4 = 3     c=4 {3,4,5}:   12/3 = 4
      c=2 {1..4}:   8/4 = 2     c=5 {4,5}:     12/2 = 6
    A zero-padded divisor-4 pool would give 3, 3, 2, 5, 3, 3 instead.
    The scalar mean is 24/6 = 4.
    """
    k = np.array([4.0, 0, 8, 0, 0, 12])
    assert np.array_equal(oracle.pool_vector_avg4(k), [4, 3, 2, 5, 4, 6])
    assert oracle.pool_scalar_mean(k)[0] == 4.0
    g = oracle.gate(k, oracle.VECTOR_AVGPOOL4)
    assert np.allclose(g, 1 / (1 + np.exp(-np.array([4, 3, 2, 5, 4, 6.0]))), rtol=0, atol=1e-15)
    assert np.allclose(oracle.gate(k, oracle.SCALAR_MEAN), 1 / (1 + math.exp(-4.0)), rtol=0, atol=1e-15)


def test_sigmoid_softmax_extremes():
    """Pin: sigmoid and softmax stay finite and exact at extreme arguments."""
    x = np.array([-800.0, -40.0, 0.0, 40.0, 800.0])
    s = oracle.sigmoid(x)
    assert np.all(np.isfinite(s)) and s[2] == 0.5 and s[4] == 1.0 and s[0] == 0.0
    assert np.allclose(s, sps.expit(x), rtol=1e-15, atol=0)
    z = np.array([1000.0, 1000.0, -1000.0])
    assert np.allclose(oracle.softmax(z), [0.5, 0.5, 0.0], rtol=0, atol=0)


@pytest.mark.parametrize("seed", range(5))
def test_gate_one_is_causal_linear_attention(seed):
    """Pin 2: with G = 1 the GRM is unnormalised causal linear attention.

    O = tril(phi(Q) phi(K)^T) V and S_T = phi(K)^T V (textbook identities).
    Catches: any decay leaking in, a missing diagonal, a wrong phi.
    """
    rng = np.random.default_rng(seed)
    T, d = 17, 8
    q = rng.standard_normal((2, T, 2, d))
    k = rng.standard_normal((2, T, 2, d))
    v = rng.standard_normal((2, T, 2, d))
    o, S, o_grm, _ = oracle.prefill(q, k, v, oracle.SCALAR_MEAN, 64, 1.0,
                                    gate_override=lambda kt: np.ones(kt.shape[:-1] + (1,)),
                                    return_parts=True)
    pq, pk = _softmax_lib(q), _softmax_lib(k)
    for b in range(2):
        for h in range(2):
            A = np.tril(pq[b, :, h] @ pk[b, :, h].T)
            assert _close(o_grm[b, :, h], A @ v[b, :, h])
            assert _close(S[b, h], pk[b, :, h].T @ v[b, :, h])
    assert _close(o, o_grm)


@pytest.mark.parametrize("n_rep", [1, 4])
def test_full_window_equals_library_causal_attention(n_rep):
    """Pin 3: window >= T makes SWA plain causal softmax attention.

    Checked against torch's scaled_dot_product_attention (float64, CPU,
    is_causal, scale 1/sqrt(d)). Catches a wrong scale or mask.
    """
    rng = np.random.default_rng(7)
    B, T, H_kv, d = 2, 23, 2, 16
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    _, _, _, o_swa = oracle.prefill(q, k, v, oracle.VECTOR_AVGPOOL4, T + 5, 0.0,
                                    return_parts=True)
    tq = torch.from_numpy(q).transpose(1, 2)                       # [B, H, T, d]
    tk = torch.from_numpy(k).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    tv = torch.from_numpy(v).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=1.0 / math.sqrt(d)).transpose(1, 2).numpy()
    assert _close(o_swa, ref, rtol=1e-12)


@pytest.mark.parametrize("n_rep", [1, 4])
def test_full_attention_equals_library_causal_attention(n_rep):
    """The hybrid's softmax layer against torch's scaled_dot_product_attention.

    float64, CPU, is_causal, scale 1/sqrt(d), the key/value head repeated for
    its n_rep query heads. Catches a wrong scale, mask or head map.
    """
    rng = np.random.default_rng(11 + n_rep)
    B, T, H_kv, d = 2, 37, 2, 16
    q = rng.standard_normal((B, T, H_kv * n_rep, d)) * 2.0
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    o = oracle.full_attention(q, k, v)
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(k).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    tv = torch.from_numpy(v).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=1.0 / math.sqrt(d)).transpose(1, 2).numpy()
    assert _close(o, ref, rtol=1e-12)


def test_full_attention_equals_unbounded_window():
    """The softmax layer is the Liger SWA with a window longer than the sequence."""
    rng = np.random.default_rng(5)
    B, T, H_kv, n_rep, d = 1, 29, 2, 2, 8
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    _, _, _, o_swa = oracle.prefill(q, k, v, oracle.SCALAR_MEAN, T, 0.0, return_parts=True)
    assert _close(oracle.full_attention(q, k, v), o_swa, rtol=1e-12)


def test_full_attention_closed_forms():
    """Equal keys give uniform weights: o_t is the running mean of v_0..v_t.
    The first token attends to itself alone: o_0 = v_0. Catches an off-by-one
    in the causal range (the mean would include one value too many or few)."""
    rng = np.random.default_rng(3)
    B, T, H_kv, n_rep, d = 2, 17, 1, 3, 8
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = np.broadcast_to(rng.standard_normal((B, 1, H_kv, d)), (B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    o = oracle.full_attention(q, k, v)
    run_mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    for h in range(H_kv * n_rep):
        assert _close(o[:, :, h], run_mean[:, :, h // n_rep], rtol=1e-12)
    o2 = oracle.full_attention(rng.standard_normal((B, T, H_kv * n_rep, d)), rng.standard_normal((B, T, H_kv, d)), v)
    for h in range(H_kv * n_rep):
        assert _close(o2[:, 0, h], v[:, 0, h // n_rep], rtol=1e-12)


@pytest.mark.parametrize("n_rep", [1, 4])
def test_full_attention_rows_pinned(n_rep):
    """Row-sampled softmax layer: every listed row equals torch's causal
    scaled_dot_product_attention (float64) at that position, and equals the
    whole-sequence oracle there. Catches a prefix off by one (t vs t + 1
    keys), rows taken from the wrong position, or a wrong head map."""
    rng = np.random.default_rng(41 + n_rep)
    B, T, H_kv, d = 2, 45, 2, 16
    q = rng.standard_normal((B, T, H_kv * n_rep, d)) * 2.0
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    rows = [0, 1, 7, 31, 32, 44, 7]
    o = oracle.full_attention_rows(q, k, v, rows)
    assert o.shape == (B, len(rows), H_kv * n_rep, d)
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(k).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    tv = torch.from_numpy(v).transpose(1, 2).repeat_interleave(n_rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=1.0 / math.sqrt(d)).transpose(1, 2).numpy()
    assert _close(o, ref[:, rows], rtol=1e-12)
    assert _close(o, oracle.full_attention(q, k, v)[:, rows], rtol=1e-12)
    with pytest.raises(ValueError):
        oracle.full_attention_rows(q, k, v, [T])


def _sink_inputs(rng, B, T, H_kv, n_rep, d, n):
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    sk = rng.standard_normal((H_kv, n, d))
    sv = rng.standard_normal((H_kv, n, d))
    return q, k, v, sk, sv


@pytest.mark.parametrize("window,n", [(4, 1), (64, 3), (7, 16)])
def test_sinks_are_prepended_tokens_bruteforce(window, n):
    """Meta-memory tokens as n extra tokens placed before the sequence that
    every query may see: an explicit [T, n + T] visibility mask and a plain
    exp / sum over it, against the oracle's SWA with sinks. Catches sinks
    that are windowed, causally masked, scaled differently or left out of
    the normaliser."""
    rng = np.random.default_rng(100 + window + n)
    B, T, H_kv, n_rep, d = 2, 19, 2, 2, 8
    q, k, v, sk, sv = _sink_inputs(rng, B, T, H_kv, n_rep, d, n)
    _, _, _, o_swa = oracle.prefill(q, k, v, oracle.VECTOR_AVGPOOL4, window, 0.0, return_parts=True,
                                    sink_k=sk, sink_v=sv)
    ref = np.zeros_like(o_swa)
    for b in range(B):
        for h in range(H_kv * n_rep):
            hk = h // n_rep
            kk = np.concatenate([sk[hk], k[b, :, hk]])        # [n + T, d]
            vv = np.concatenate([sv[hk], v[b, :, hk]])
            for t in range(T):
                vis = np.array([j < n or (t - window < j - n <= t) for j in range(n + T)])
                w = np.exp(kk @ q[b, t, h] / math.sqrt(d)) * vis
                ref[b, t, h] = (w / w.sum()) @ vv
    assert _close(o_swa, ref, rtol=1e-12)


def test_sinks_zero_keys_and_values_closed_form():
    """n sinks with zero keys and values add e^0 = 1 each to the softmax
    normaliser and nothing to the numerator: o_sink = o_plain * Z / (Z + n),
    Z = sum over the window of e^{q.k/sqrt(d)}."""
    rng = np.random.default_rng(9)
    B, T, H_kv, n_rep, d, n, window = 1, 15, 1, 2, 8, 5, 6
    q, k, v, _, _ = _sink_inputs(rng, B, T, H_kv, n_rep, d, n)
    zk, zv = np.zeros((H_kv, n, d)), np.zeros((H_kv, n, d))
    _, _, _, o_plain = oracle.prefill(q, k, v, oracle.SCALAR_MEAN, window, 0.0, return_parts=True)
    _, _, _, o_sink = oracle.prefill(q, k, v, oracle.SCALAR_MEAN, window, 0.0, return_parts=True,
                                     sink_k=zk, sink_v=zv)
    for t in range(T):
        lo = max(0, t - window + 1)
        for h in range(H_kv * n_rep):
            Z = np.exp(k[0, lo:t + 1, h // n_rep] @ q[0, t, h] / math.sqrt(d)).sum()
            assert _close(o_sink[0, t, h], o_plain[0, t, h] * Z / (Z + n), rtol=1e-12)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
def test_sinks_decode_continues_prefill(mode):
    """Prefill(T0) then decode steps with the same sinks equals prefill(T0 + n)."""
    rng = np.random.default_rng(21)
    B, T, H_kv, n_rep, d, n, window = 2, 13, 2, 2, 8, 4, 5
    q, k, v, sk, sv = _sink_inputs(rng, B, T, H_kv, n_rep, d, n)
    T0 = 8
    o_full, S_full = oracle.prefill(q, k, v, mode, window, 0.5, sink_k=sk, sink_v=sv)
    _, S = oracle.prefill(q[:, :T0], k[:, :T0], v[:, :T0], mode, window, 0.5, sink_k=sk, sink_v=sv)
    rk, rv, pos = oracle.ring_fill(k[:, :T0], v[:, :T0], window)
    for t in range(T0, T):
        o, S, rk, rv, pos = oracle.decode_step(q[:, t], k[:, t], v[:, t], S, rk, rv, pos, mode, 0.5,
                                               sink_k=sk, sink_v=sv)
        assert _close(o, o_full[:, t], rtol=1e-11)
    assert _close(S, S_full, rtol=1e-11)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
@pytest.mark.parametrize("n_rep,window,alpha", [(1, 1, 0.5), (2, 3, 0.3), (2, 64, 0.8)])
def test_backward_matches_central_differences(mode, n_rep, window, alpha):
    """Every entry of dq, dk, dv against central differences of sum(o * W)
    on the float64 forward (h = 1e-6). Catches any dropped term of the
    chain rule (adjoint decay, gate, pool transpose, softmax Jacobians,
    window range)."""
    rng = np.random.default_rng(50 + 7 * n_rep + window + mode)
    B, T, H_kv, d = 1, 6, 1, 4
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    W = rng.standard_normal((B, T, H_kv * n_rep, d))
    dq, dk, dv = oracle.prefill_backward(q, k, v, W, mode, window, alpha)

    def loss(qq, kk, vv):
        return float(np.sum(oracle.prefill(qq, kk, vv, mode, window, alpha)[0] * W))

    h = 1e-6
    for name, X, G in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(X.shape):
            args = {"qq": q, "kk": k, "vv": v}
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args[name * 2] = Xp
            lp = loss(**args)
            args[name * 2] = Xm
            lm = loss(**args)
            assert abs((lp - lm) / (2 * h) - G[idx]) <= 1e-6, (name, idx)


@pytest.mark.parametrize("n_rep", [1, 2])
def test_backward_full_window_is_library_attention_gradient(n_rep):
    """alpha = 0 and a window longer than the sequence: the gradients of plain
    causal softmax attention, from torch autograd of scaled_dot_product_attention
    in float64."""
    rng = np.random.default_rng(70 + n_rep)
    B, T, H_kv, d = 2, 11, 2, 8
    q = rng.standard_normal((B, T, H_kv * n_rep, d))
    k = rng.standard_normal((B, T, H_kv, d))
    v = rng.standard_normal((B, T, H_kv, d))
    W = rng.standard_normal((B, T, H_kv * n_rep, d))
    dq, dk, dv = oracle.prefill_backward(q, k, v, W, oracle.SCALAR_MEAN, T + 3, 0.0)
    tq = torch.from_numpy(q).transpose(1, 2).requires_grad_()
    tk = torch.from_numpy(k).transpose(1, 2).requires_grad_()
    tv = torch.from_numpy(v).transpose(1, 2).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(n_rep, dim=1), tv.repeat_interleave(n_rep, dim=1), is_causal=True,
        scale=1.0 / math.sqrt(d))
    (o * torch.from_numpy(W).transpose(1, 2)).sum().backward()
    assert _close(dq, tq.grad.transpose(1, 2).numpy(), rtol=1e-12)
    assert _close(dk, tk.grad.transpose(1, 2).numpy(), rtol=1e-12)
    assert _close(dv, tv.grad.transpose(1, 2).numpy(), rtol=1e-12)


def test_alpha_is_affine_and_endpoints():
    """Pin 4: o(alpha) = alpha o(1) + (1-alpha) o(0); alpha=1 pure GRM, 0 pure SWA."""
    x = prefill_inputs(B=1, T=40, H_q=4, H_kv=2, d=8, dtype="f32", seed=3)
    o1, S1 = oracle.prefill(x["q"], x["k"], x["v"], oracle.VECTOR_AVGPOOL4, 9, 1.0)
    o0, S0 = oracle.prefill(x["q"], x["k"], x["v"], oracle.VECTOR_AVGPOOL4, 9, 0.0)
    oa, Sa, og, osw = oracle.prefill(x["q"], x["k"], x["v"], oracle.VECTOR_AVGPOOL4, 9, 0.3,
                                     return_parts=True)
    assert _close(oa, 0.3 * o1 + 0.7 * o0)
    assert _close(o1, og) and _close(o0, osw)
    assert np.array_equal(S1, S0) and np.array_equal(S1, Sa)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
@pytest.mark.parametrize("T0,n,window", [(5, 7, 4), (1, 12, 64), (70, 3, 64), (64, 1, 64), (3, 5, 1)])
def test_decode_continues_prefill(mode, T0, n, window):
    """Pin 5: prefill(T0) then n decode steps == prefill(T0 + n).

    Checks the outputs of the last n tokens, the final state, the ring
    contents (the last `window` tokens, slot t mod window) and pos.
    """
    x = prefill_inputs(B=2, T=T0 + n, H_q=4, H_kv=2, d=8, dtype="f32", seed=11)
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full = oracle.prefill(q, k, v, mode, window, 0.4)
    _, S = oracle.prefill(q[:, :T0], k[:, :T0], v[:, :T0], mode, window, 0.4)
    rk, rv, pos = oracle.ring_fill(k[:, :T0], v[:, :T0], window)
    for i in range(n):
        t = T0 + i
        o_t, S, rk, rv, pos = oracle.decode_step(q[:, t], k[:, t], v[:, t], S, rk, rv, pos, mode, 0.4)
        assert _close(o_t, o_full[:, t])
    assert _close(S, S_full)
    rk_ref, rv_ref, pos_ref = oracle.ring_fill(k, v, window)
    assert np.array_equal(rk, rk_ref) and np.array_equal(rv, rv_ref) and np.array_equal(pos, pos_ref)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
@pytest.mark.parametrize("T1,T2,window", [(0, 9, 4), (5, 7, 4), (1, 12, 64), (70, 3, 64), (3, 5, 1), (40, 30, 17)])
def test_prefill_continue_is_concatenation(mode, T1, T2, window):
    """Pin 5 for the continuation: prefill(T1), ring after it, then T2 tokens
    in one continuation call == prefill(T1 + T2): outputs of the last T2
    tokens, the final state, the ring (the last `window` tokens) and pos.
    T1 = 0 starts from a zero state and an empty ring."""
    x = prefill_inputs(B=2, T=T1 + T2, H_q=4, H_kv=2, d=8, dtype="f32", seed=23)
    q, k, v = x["q"], x["k"], x["v"]
    o_full, S_full = oracle.prefill(q, k, v, mode, window, 0.35)
    if T1 > 0:
        _, S0 = oracle.prefill(q[:, :T1], k[:, :T1], v[:, :T1], mode, window, 0.35)
    else:
        S0 = np.zeros((2, 2, 8, 8))
    rk, rv, pos = oracle.ring_fill(k[:, :T1], v[:, :T1], window)
    o, S, rk, rv, pos = oracle.prefill_continue(q[:, T1:], k[:, T1:], v[:, T1:], S0, rk, rv, pos, mode, 0.35)
    assert _close(o, o_full[:, T1:])
    assert _close(S, S_full)
    rk_ref, rv_ref, pos_ref = oracle.ring_fill(k, v, window)
    assert np.array_equal(rk, rk_ref) and np.array_equal(rv, rv_ref) and np.array_equal(pos, pos_ref)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
@pytest.mark.parametrize("c", [0.0, -1.5, 2.0])
def test_closed_form_constant_key(mode, c):
    """Pin 6: k_t = c*1, v_t = v: a geometric series, derived by hand.

    phi(k) = 1/d, every pooled value is c so g = sigmoid(c) in both modes, and
      S_t = (1/d) 1 v^T (1 - g^{t+1}) / (1 - g)
      o_grm,t = (1/d) (1 - g^{t+1}) / (1 - g) v   for any q (phi(q) sums to 1)
      o_swa,t = v (equal logits over identical values).
    """
    T, d, alpha = 50, 8, 0.5
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, T, 2, d)) * 3
    k = np.full((1, T, 1, d), c)
    vv = rng.standard_normal(d)
    v = np.broadcast_to(vv, (1, T, 1, d)).copy()
    o, S = oracle.prefill(q, k, v, mode, 64, alpha)
    g = 1.0 / (1.0 + math.exp(-c))
    for t in range(T):
        geo = (1 - g ** (t + 1)) / (1 - g)
        ref = alpha * geo / d * vv + (1 - alpha) * vv
        assert np.allclose(o[0, t, 0], ref, rtol=1e-12, atol=1e-13)
        assert np.allclose(o[0, t, 1], ref, rtol=1e-12, atol=1e-13)
    geo = (1 - g ** T) / (1 - g)
    assert np.allclose(S[0, 0], np.outer(np.full(d, 1.0 / d), vv) * geo, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
def test_key_shift_moves_only_the_gate(mode):
    """Pin 7: k -> k + c*1 leaves phi(k) and SWA unchanged and shifts every pooled value by c.

    Catches a pool whose divisor is not the in-range count (then the shift
    would not be uniform at the edges) and phi applied with a temperature.
    """
    rng = np.random.default_rng(9)
    T, d, c = 30, 8, 0.75
    q = rng.standard_normal((1, T, 2, d))
    k = rng.standard_normal((1, T, 2, d))
    v = rng.standard_normal((1, T, 2, d))
    pool = oracle.pool_scalar_mean if mode == oracle.SCALAR_MEAN else oracle.pool_vector_avg4
    assert np.allclose(pool(k + c), pool(k) + c, rtol=0, atol=1e-14)
    o_a, S_a, og_a, os_a = oracle.prefill(q, k, v, mode, 16, 0.5, return_parts=True)
    o_b, S_b, og_b, os_b = oracle.prefill(q, k + c, v, mode, 16, 0.5, return_parts=True,
                                          gate_override=lambda kt: oracle.gate(kt - c, mode))
    assert _close(os_a, os_b) and _close(og_a, og_b) and _close(S_a, S_b)


def test_window_one_and_single_token():
    """Pin 8: window 1 gives o_swa,t = v_t; T = 1 gives o = (alpha phi(q).phi(k) + 1 - alpha) v."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 12, 2, 8))
    k = rng.standard_normal((1, 12, 1, 8))
    v = rng.standard_normal((1, 12, 1, 8))
    _, _, _, o_swa = oracle.prefill(q, k, v, oracle.VECTOR_AVGPOOL4, 1, 0.5, return_parts=True)
    assert _close(o_swa[0, :, 0], v[0, :, 0]) and _close(o_swa[0, :, 1], v[0, :, 0])
    o, S = oracle.prefill(q[:, :1], k[:, :1], v[:, :1], oracle.SCALAR_MEAN, 64, 0.3)
    for h in range(2):
        dot = float(_softmax_lib(q[0, 0, h]) @ _softmax_lib(k[0, 0, 0]))
        assert _close(o[0, 0, h], (0.3 * dot + 0.7) * v[0, 0, 0])
    # S_1 = phi(k_0)^T v_0 (S_0 = 0, so the gate of token 0 has no effect)
    assert _close(S[0, 0], np.outer(_softmax_lib(k[0, 0, 0]), v[0, 0, 0]))


@pytest.mark.parametrize("mode", [oracle.SCALAR_MEAN, oracle.VECTOR_AVGPOOL4])
def test_gqa_equals_repeated_mha_and_batch_independence(mode):
    """Pin 9: GQA equals MHA on k, v repeated per group (contiguous groups);
    batch elements are independent; a d_v permutation is equivariant."""
    x = prefill_inputs(B=3, T=20, H_q=6, H_kv=2, d=8, dtype="f32", seed=21)
    q, k, v = x["q"], x["k"], x["v"]
    o, S = oracle.prefill(q, k, v, mode, 6, 0.5)
    o_m, S_m = oracle.prefill(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), mode, 6, 0.5)
    assert _close(o, o_m)
    for h in range(6):
        assert _close(S_m[:, h], S[:, h // 3])
    o_1, S_1 = oracle.prefill(q[1:2], k[1:2], v[1:2], mode, 6, 0.5)
    assert _close(o[1:2], o_1) and _close(S[1:2], S_1)
    perm = np.random.default_rng(0).permutation(8)
    o_p, S_p = oracle.prefill(q, k, v[..., perm], mode, 6, 0.5)
    # q and k are untouched so the gate, phi and SWA weights are unchanged
    o_pm, _ = oracle.prefill(q, k, v, mode, 6, 0.5)
    assert _close(o_p, o_pm[..., perm]) and _close(S_p, S[..., perm])


def test_bf16_storage_is_exact_in_float64():
    """Inputs stored as bf16 widen exactly; the oracle sees the same values."""
    x = prefill_inputs(B=1, T=4, H_q=2, H_kv=1, d=8, dtype="bf16", seed=2)
    assert np.array_equal(round_to_bf16(x["q"]), x["q"])


def test_golden_regression_fixture():
    """The oracle still reproduces the committed fixture (written by tests/golden/make_golden.py)."""
    import json
    import os
    from synth import prefill_inputs as gen
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_prefill_small.json")
    with open(path) as f:
        fx = json.load(f)
    x = gen(**fx["inputs"])
    o, S = oracle.prefill(x["q"], x["k"], x["v"], fx["gate_mode"], fx["window"], fx["alpha"])
    assert np.allclose(o.ravel()[fx["o_index"]], fx["o_values"], rtol=1e-13, atol=1e-15)
    assert np.allclose(S.ravel()[fx["S_index"]], fx["S_values"], rtol=1e-13, atol=1e-15)
