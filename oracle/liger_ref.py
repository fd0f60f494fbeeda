"""Float64 CPU oracle of the Liger Attention layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it, and
it shares no code, constants or helpers with the GPU library.

What it computes, and where the pages state it
----------------------------------------------
Sources (the page titles and sections are cited, nothing else):
  [Notes]  paper-notes page "Liger: Linearizing Large Language Models to Gated
           Recurrent Structures" (ICML2025, model_compression), sections
           "核心思想：Key 投影复用构建门控" (gate from the key projection),
           "统一的门控线性循环框架" (unified gated linear recurrence) and
           "Liger Attention：层内混合注意力" (intra-layer hybrid).
  [News]   Japanese news article on Liger (Shanghai AI Lab, ICML 2025),
           section "手法の説明" (softmax as the feature map on Q and K; the
           parameter-free pooling gate) and "ハイブリッドメカニズム：Liger
           Attention".

  gate     G_t = f(k_t) with f a parameter-free pooling of the key
           ([Notes] gate equation; [News] 手法の説明). The pages say only
           "pooling, e.g. mean"; the two pooled gates below are the readings
           fixed for this implementation, each squashed by a sigmoid so that
           0 < g < 1:
             scalar : g_t = sigmoid(mean_c k_t[c]), applied to every entry of S
             vector : g_t[c] = sigmoid(mean{k_t[m] : m in [c-1, c+2], 0<=m<d}),
                      applied to row c (the d_k index) of S; the divisor is the
                      number of in-range channels (4 inside, 3 at c=0 and c=d-2,
                      2 at c=d-1).
  feature  phi = softmax over the head dimension, applied to q and to k
  map      separately, without a temperature ([Notes] recurrence section;
           [News] 手法の説明).
  GRM      S_t = G_t * S_{t-1} + phi(k_t)^T v_t ;  o_t = phi(q_t) S_t
           ([Notes] unified recurrence; the printed transpose placement is
           garbled, phi(k_t)^T v_t is read as an outer product d_k x d_v).
           S_0 = 0. The output uses the state that already includes token t.
  SWA      causal softmax attention of raw q over the last `window` keys,
           the current key included, with scale 1/sqrt(d) ([Notes] hybrid
           section: window 64).
  mix      o_t = alpha * GRM + (1 - alpha) * SWA, alpha + beta = 1, default
           0.5 ([Notes] hybrid section).
  GQA      query head h reads key/value head h // (H_q // H_kv); the state is
           kept per key/value head (the pages are silent; the plainest reading).

sinks    meta-memory tokens (Japanese summary page of Lizard, section
           "アンカーウィンドウアテンション"): n extra key/value pairs per key/value
           head that every window's softmax also sees; they act as attention
           sinks. The page gives no formula; the reading fixed here: the n
           pairs are prepended to the window of every query, with the same
           1/sqrt(d) scale and no causal or window mask, and they do not enter
           the recurrence. Their values are synthetic inputs.
full     the hybrid's standard softmax attention layer (one after every few
attention Liger blocks: [Notes] section "Liger 整体架构", inter-layer hybrid):
           causal softmax attention of raw q over every earlier key, the
           current one included, scale 1/sqrt(d), the same GQA head map.

Decode keeps (S, ring of the last `window` keys/values, pos) per sequence: the
fixed-size state that linear decoding carries instead of a growing KV cache
([News] 実験分析: constant memory at long context). Token t of a sequence
lives in ring slot t mod window.

Everything is float64. Inputs are widened exactly (bf16 and fp32 values are
exact in float64). Nothing is rounded on the way out.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against a brute-force parallel form, textbook reductions (G = 1, w >= T),
a library attention routine, closed forms and hand-derived fixtures.
"""
from __future__ import annotations

import numpy as np

SCALAR_MEAN = 0
VECTOR_AVGPOOL4 = 1


def sigmoid(x):
    """1 / (1 + e^{-x}), evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def softmax(x, axis=-1):
    """e^{x - max x} / sum e^{x - max x} along `axis` (the exact definition)."""
    x = np.asarray(x, dtype=np.float64)
    z = np.exp(x - np.max(x, axis=axis, keepdims=True))
    return z / np.sum(z, axis=axis, keepdims=True)


def pool_scalar_mean(k):
    """Mean over the head dimension; result keeps a length-1 last axis."""
    k = np.asarray(k, dtype=np.float64)
    return np.mean(k, axis=-1, keepdims=True)


def pool_vector_avg4(k):
    """Per-channel average of the in-range channels c-1 .. c+2 (kernel 4, 'same')."""
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[-1]
    out = np.empty_like(k)
    for c in range(d):
        lo, hi = max(0, c - 1), min(d, c + 3)
        out[..., c] = np.mean(k[..., lo:hi], axis=-1)
    return out


def gate(k, gate_mode):
    """g = sigmoid(pool(k)) on the raw key (before phi).

    Returns an array whose last axis broadcasts over the d_k rows of S:
    length 1 for the scalar gate, length d for the vector gate.
    """
    if gate_mode == SCALAR_MEAN:
        return sigmoid(pool_scalar_mean(k))
    if gate_mode == VECTOR_AVGPOOL4:
        return sigmoid(pool_vector_avg4(k))
    raise ValueError(f"unknown gate mode {gate_mode!r}")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _with_sinks(kw, vw, sink_k, sink_v, lead):
    """Prepend the sink keys/values ([H_kv, n, d]) to a window's keys [..., d, L]
    and values [..., L, d]; `lead` leading batch axes are broadcast."""
    if sink_k is None:
        return kw, vw
    sk, sv = _f64(sink_k), _f64(sink_v)
    skT = np.broadcast_to(sk.transpose(0, 2, 1), kw.shape[:lead] + sk.transpose(0, 2, 1).shape)
    svb = np.broadcast_to(sv, vw.shape[:lead] + sv.shape)
    return np.concatenate([skT, kw], axis=-1), np.concatenate([svb, vw], axis=-2)


def prefill(q, k, v, gate_mode, window, alpha, *, gate_override=None,
            S0=None, return_parts=False, sink_k=None, sink_v=None):
    """Token-by-token Liger Attention over whole sequences.

    q: [B, T, H_q, d]; k, v: [B, T, H_kv, d]. Returns (o [B, T, H_q, d],
    S_T [B, H_kv, d, d]); with return_parts, also (o_grm, o_swa).
    `gate_override(k_t) -> g_t` replaces the pooled gate (test hook).
    `S0` is the initial state (zero when None). `sink_k`, `sink_v`
    ([H_kv, n, d]) are meta-memory tokens prepended to every window.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    n_rep = H_q // H_kv
    if not 1 <= window:
        raise ValueError("window must be >= 1")
    scale = 1.0 / np.sqrt(d)

    phi_q = softmax(q).reshape(B, T, H_kv, n_rep, d)
    phi_k = softmax(k)
    qg = q.reshape(B, T, H_kv, n_rep, d)
    S = np.zeros((B, H_kv, d, d)) if S0 is None else _f64(S0).copy()
    o_grm = np.empty((B, T, H_kv, n_rep, d))
    o_swa = np.empty((B, T, H_kv, n_rep, d))
    for t in range(T):
        g = gate_override(k[:, t]) if gate_override is not None else gate(k[:, t], gate_mode)
        g = np.broadcast_to(_f64(g), (B, H_kv, d))
        # S_t = G_t (.) S_{t-1} + phi(k_t)^T v_t  (rows: d_k, columns: d_v)
        S = g[..., :, None] * S + phi_k[:, t, :, :, None] * v[:, t, :, None, :]
        # o_t = phi(q_t) S_t, with S_t already holding token t
        o_grm[:, t] = np.matmul(phi_q[:, t], S)
        # causal window of `window` keys ending at t (inclusive)
        lo = max(0, t - window + 1)
        kw = k[:, lo:t + 1].transpose(0, 2, 3, 1)          # [B, H_kv, d, L]
        vw = v[:, lo:t + 1].transpose(0, 2, 1, 3)          # [B, H_kv, L, d]
        kw, vw = _with_sinks(kw, vw, sink_k, sink_v, 1)    # sinks first: [.., n + L]
        p = softmax(np.matmul(qg[:, t], kw) * scale)       # [B, H_kv, n_rep, n + L]
        o_swa[:, t] = np.matmul(p, vw)
    o_grm = o_grm.reshape(B, T, H_q, d)
    o_swa = o_swa.reshape(B, T, H_q, d)
    o = alpha * o_grm + (1.0 - alpha) * o_swa
    if return_parts:
        return o, S, o_grm, o_swa
    return o, S


def ring_fill(k, v, window):
    """Decode state after a prompt: token t sits in slot t mod window.

    k, v: [B, T, H_kv, d]. Returns ring_k, ring_v [B, H_kv, window, d] and
    pos [B] (= T). Slots that hold no token (T < window) are zero.
    """
    k, v = np.asarray(k), np.asarray(v)
    B, T, H_kv, d = k.shape
    ring_k = np.zeros((B, H_kv, window, d), dtype=k.dtype)
    ring_v = np.zeros((B, H_kv, window, d), dtype=v.dtype)
    for t in range(max(0, T - window), T):
        ring_k[:, :, t % window] = k[:, t]
        ring_v[:, :, t % window] = v[:, t]
    return ring_k, ring_v, np.full((B,), T, dtype=np.int64)


def decode_step(q, k, v, S, ring_k, ring_v, pos, gate_mode, alpha, *,
                gate_override=None, return_parts=False, sink_k=None, sink_v=None):
    """One token per sequence from the fixed-size decode state.

    q: [N, H_q, d]; k, v: [N, H_kv, d]; S: [N, H_kv, d, d];
    ring_k, ring_v: [N, H_kv, window, d]; pos: [N] tokens already consumed.
    Returns (o [N, H_q, d], S', ring_k', ring_v', pos + 1). The new token is
    token number pos[n]; it is written to slot pos[n] mod window and the
    window covers tokens max(0, pos-window+1) .. pos (the new one included),
    after the meta-memory tokens `sink_k`, `sink_v` ([H_kv, n, d]) if given.
    """
    q, kf, vf = _f64(q), _f64(k), _f64(v)
    N, H_q, d = q.shape
    H_kv = kf.shape[1]
    n_rep = H_q // H_kv
    window = ring_k.shape[2]
    pos = np.asarray(pos, dtype=np.int64)
    scale = 1.0 / np.sqrt(d)

    g = gate_override(kf) if gate_override is not None else gate(kf, gate_mode)
    g = np.broadcast_to(_f64(g), (N, H_kv, d))
    S_new = g[..., :, None] * _f64(S) + softmax(kf)[..., :, None] * vf[..., None, :]
    o_grm = np.matmul(softmax(q).reshape(N, H_kv, n_rep, d), S_new)

    ring_k_new = np.array(ring_k, copy=True)
    ring_v_new = np.array(ring_v, copy=True)
    o_swa = np.empty((N, H_kv, n_rep, d))
    qg = q.reshape(N, H_kv, n_rep, d)
    for n in range(N):
        p_n = int(pos[n])
        ring_k_new[n, :, p_n % window] = k[n]
        ring_v_new[n, :, p_n % window] = v[n]
        toks = range(max(0, p_n - window + 1), p_n + 1)
        slots = [t % window for t in toks]
        kw = _f64(ring_k_new[n][:, slots]).transpose(0, 2, 1)   # [H_kv, d, L]
        vw = _f64(ring_v_new[n][:, slots])                      # [H_kv, L, d]
        kw, vw = _with_sinks(kw, vw, sink_k, sink_v, 0)
        p = softmax(np.matmul(qg[n], kw) * scale)
        o_swa[n] = np.matmul(p, vw)
    o_grm = o_grm.reshape(N, H_q, d)
    o_swa = o_swa.reshape(N, H_q, d)
    o = alpha * o_grm + (1.0 - alpha) * o_swa
    out = (o, S_new, ring_k_new, ring_v_new, pos + 1)
    if return_parts:
        return out + (o_grm, o_swa)
    return out


def prefill_continue(q, k, v, S0, ring_k, ring_v, pos, gate_mode, alpha, *, gate_override=None,
                     sink_k=None, sink_v=None):
    """T more tokens per sequence after `pos` already consumed ones.

    The plain definition: T successive decode steps from the fixed-size state
    (S0, ring of the last `window` keys/values, pos), the same state decoding
    carries ([News] 実験分析). q: [B, T, H_q, d]; k, v: [B, T, H_kv, d];
    S0: [B, H_kv, d, d]; ring_k, ring_v: [B, H_kv, window, d]; pos: [B].
    Returns (o [B, T, H_q, d], S_T, ring_k', ring_v', pos + T).
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    B, T, H_q, d = q.shape
    S = _f64(S0)
    rk, rv = np.array(ring_k, copy=True), np.array(ring_v, copy=True)
    p = np.asarray(pos, dtype=np.int64).copy()
    o = np.empty((B, T, H_q, d))
    for t in range(T):
        o[:, t], S, rk, rv, p = decode_step(q[:, t], k[:, t], v[:, t], S, rk, rv, p, gate_mode, alpha,
                                            gate_override=gate_override, sink_k=sink_k, sink_v=sink_v)
    return o, S, rk, rv, p



def full_attention(q, k, v):
    """Causal softmax attention over all earlier keys (the hybrid's softmax layer).

    o_t = sum_{j <= t} softmax_j(q_t . k_j / sqrt(d)) v_j for every query head,
    query head h reading key/value head h // (H_q // H_kv) ([Notes] section
    "Liger 整体架构": a standard softmax attention block between Liger blocks).
    q: [B, T, H_q, d]; k, v: [B, T, H_kv, d]. Returns o [B, T, H_q, d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    n_rep = H_q // H_kv
    scale = 1.0 / np.sqrt(d)
    qg = q.reshape(B, T, H_kv, n_rep, d)
    o = np.empty((B, T, H_kv, n_rep, d))
    for t in range(T):
        kw = k[:, :t + 1].transpose(0, 2, 3, 1)            # [B, H_kv, d, t+1]
        vw = v[:, :t + 1].transpose(0, 2, 1, 3)            # [B, H_kv, t+1, d]
        p = softmax(np.matmul(qg[:, t], kw) * scale)       # [B, H_kv, n_rep, t+1]
        o[:, t] = np.matmul(p, vw)
    return o.reshape(B, T, H_q, d)


def full_attention_rows(q, k, v, rows):
    """The same causal softmax attention as full_attention, for chosen query
    positions only: o[:, i] = sum_{j <= rows[i]} softmax_j(q_t . k_j / sqrt(d)) v_j
    with t = rows[i], each from its whole causal prefix.

    q: [B, T, H_q, d]; k, v: [B, T, H_kv, d]; rows: positions in [0, T).
    Returns [B, len(rows), H_q, d]. This is the definition restricted to the
    listed rows (sequences too long for the whole-sequence loop).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    n_rep = H_q // H_kv
    scale = 1.0 / np.sqrt(d)
    rows = [int(t) for t in rows]
    if any(t < 0 or t >= T for t in rows):
        raise ValueError("rows must lie in [0, T)")
    o = np.empty((B, len(rows), H_kv, n_rep, d))
    for i, t in enumerate(rows):
        qt = q[:, t].reshape(B, H_kv, n_rep, d)
        kw = k[:, :t + 1].transpose(0, 2, 3, 1)            # [B, H_kv, d, t+1]
        vw = v[:, :t + 1].transpose(0, 2, 1, 3)            # [B, H_kv, t+1, d]
        p = softmax(np.matmul(qt, kw) * scale)             # [B, H_kv, n_rep, t+1]
        o[:, i] = np.matmul(p, vw)
    return o.reshape(B, len(rows), H_q, d)


def prefill_backward(q, k, v, dO, gate_mode, window, alpha):
    """Gradients (dq, dk, dv) of sum(o * dO) for o = prefill(q, k, v, ...) from a zero state.

    The chain rule through each step of the definition, in reverse token
    order ([Notes] unified recurrence and Liger Attention sections):
      GRM  o_t = phi(q_t) S_t, S_t = G_t (.) S_{t-1} + phi(k_t)^T v_t, adjoint
           dS_t = sum_h phi(q_t^h)^T (alpha dO_t^h) + G_{t+1} (.) dS_{t+1};
           dphi(q_t^h) = S_t (alpha dO_t^h), dphi(k_t) = dS_t v_t,
           dv_t += phi(k_t) dS_t, dG_t = dS_t (.) S_{t-1} (summed over the
           entries G_t scales: all of S for the scalar gate, row c for g[c]).
      gate g = sigmoid(pool(k)): ds = dg g (1 - g), then the pool's transpose.
      phi  softmax: dx = phi (.) (dphi - <dphi, phi>).
      SWA  p = softmax(q k^T / sqrt(d)) over the window, o = p v:
           dp = (1 - alpha) dO v^T, dz = p (.) (dp - <dp, p>),
           dq += dz k / sqrt(d), dk += dz^T q / sqrt(d), dv += p^T (1 - alpha) dO.
    q, dO: [B, T, H_q, d]; k, v: [B, T, H_kv, d]. Returns float64 arrays.
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    n_rep = H_q // H_kv
    scale = 1.0 / np.sqrt(d)
    phi_q = softmax(q).reshape(B, T, H_kv, n_rep, d)
    phi_k = softmax(k)
    dOg = dO.reshape(B, T, H_kv, n_rep, d)
    qg = q.reshape(B, T, H_kv, n_rep, d)
    # forward: gates and every state (the adjoint needs S_{t-1})
    if gate_mode == SCALAR_MEAN:
        s_pre = pool_scalar_mean(k)                       # [B, T, H_kv, 1]
    else:
        s_pre = pool_vector_avg4(k)                       # [B, T, H_kv, d]
    g = sigmoid(s_pre)
    gS = np.broadcast_to(g, (B, T, H_kv, d))
    S_all = np.zeros((T + 1, B, H_kv, d, d))              # S_all[t + 1] = S_t
    for t in range(T):
        S_all[t + 1] = gS[:, t, :, :, None] * S_all[t] + phi_k[:, t, :, :, None] * v[:, t, :, None, :]
    d_phi_q = np.zeros((B, T, H_kv, n_rep, d))
    d_phi_k = np.zeros((B, T, H_kv, d))
    dv = np.zeros((B, T, H_kv, d))
    dg = np.zeros_like(g)
    dS = np.zeros((B, H_kv, d, d))
    for t in range(T - 1, -1, -1):
        if t + 1 < T:
            dS = gS[:, t + 1, :, :, None] * dS
        dS = dS + np.einsum("bhrc,bhre->bhce", phi_q[:, t], alpha * dOg[:, t])
        S_t = S_all[t + 1]
        d_phi_q[:, t] = np.einsum("bhce,bhre->bhrc", S_t, alpha * dOg[:, t])
        d_phi_k[:, t] = np.einsum("bhce,bhe->bhc", dS, v[:, t])
        dv[:, t] += np.einsum("bhc,bhce->bhe", phi_k[:, t], dS)
        prod = dS * S_all[t]                              # dS_t (.) S_{t-1}
        if gate_mode == SCALAR_MEAN:
            dg[:, t] = prod.sum(axis=(-1, -2))[..., None]
        else:
            dg[:, t] = prod.sum(axis=-1)
    # gate: sigmoid, then the pool's transpose
    ds = dg * g * (1.0 - g)
    dk = np.zeros((B, T, H_kv, d))
    if gate_mode == SCALAR_MEAN:
        dk += ds / d
    else:
        for c in range(d):
            lo, hi = max(0, c - 1), min(d, c + 3)
            dk[..., lo:hi] += ds[..., c:c + 1] / (hi - lo)
    # softmax feature maps
    dq = (phi_q * (d_phi_q - np.sum(d_phi_q * phi_q, axis=-1, keepdims=True))).reshape(B, T, H_q, d)
    dk += phi_k * (d_phi_k - np.sum(d_phi_k * phi_k, axis=-1, keepdims=True))
    dq = dq.reshape(B, T, H_kv, n_rep, d)
    # sliding-window softmax attention
    for t in range(T):
        lo = max(0, t - window + 1)
        kw = k[:, lo:t + 1]                                # [B, L, H_kv, d]
        vw = v[:, lo:t + 1]
        z = np.einsum("bhrc,blhc->bhrl", qg[:, t], kw) * scale
        p = softmax(z)                                     # [B, H_kv, n_rep, L]
        do = (1.0 - alpha) * dOg[:, t]                     # [B, H_kv, n_rep, d]
        dp = np.einsum("bhre,blhe->bhrl", do, vw)
        dz = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
        dq[:, t] += np.einsum("bhrl,blhc->bhrc", dz, kw) * scale
        dk[:, lo:t + 1] += np.einsum("bhrl,bhrc->blhc", dz, qg[:, t]) * scale
        dv[:, lo:t + 1] += np.einsum("bhrl,bhre->blhe", p, do)
    return dq.reshape(B, T, H_q, d), dk, dv
