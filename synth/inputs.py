"""Seeded synthetic workloads for the Liger Attention layer.

Every tensor is drawn from NumPy's PCG64 generator with a fixed seed, in a
fixed order, so the GPU side and the float64 reference side see the same
bits. Values stored as bfloat16 are rounded once, round-to-nearest-even,
from the float32 draw; those bf16 bit patterns are the canonical input.

Shapes follow the Llama-3 head geometry (32 query heads, 8 key/value heads,
head size 128 for 8B; head size 64 for 1B). No model weights or datasets
are involved: the activations are standard normal stand-ins.

Layouts (row-major, contiguous):
  q, o : [B, T, H_q, d]
  k, v : [B, T, H_kv, d]
  S    : [B, H_kv, d_k, d_v]   float32
  ring : [N, H_kv, window, d]
"""
from __future__ import annotations

import numpy as np

# Named workloads. `seed` is the workload's own index; every draw below uses
# Generator(PCG64(seed)) unless stated otherwise.
CONFIGS = {
    # fp32 correctness workload: scalar gate, no GQA.
    "prefill_fp32_b1_h2_t256_d64": dict(
        kind="prefill", B=1, T=256, H_q=2, H_kv=2, d=64, dtype="f32",
        gate="scalar", window=64, alpha=0.5, seed=1, outlier_frac=0.0),
    # Llama-3.2-1B head geometry, vector gate.
    "prefill_1b_b4_t2048_d64": dict(
        kind="prefill", B=4, T=2048, H_q=32, H_kv=8, d=64, dtype="bf16",
        gate="vector", window=64, alpha=0.5, seed=2, outlier_frac=0.0),
    # Llama-3-8B head geometry, scalar gate.
    "prefill_8b_b1_t8192_d128": dict(
        kind="prefill", B=1, T=8192, H_q=32, H_kv=8, d=128, dtype="bf16",
        gate="scalar", window=64, alpha=0.5, seed=3, outlier_frac=0.0),
    # Llama-3-8B decode: 64 sequences, 1024 single-token steps, vector gate.
    "decode_8b_n64_d128": dict(
        kind="decode", N=64, H_q=32, H_kv=8, d=128, dtype="bf16",
        gate="vector", window=64, alpha=0.5, seed=4, steps=1024,
        pos0=32768, state_std=0.1),
    # Long context at 8B geometry with 1% of key rows scaled by 8.
    "prefill_8b_b1_t32768_d128_outliers": dict(
        kind="prefill", B=1, T=32768, H_q=32, H_kv=8, d=128, dtype="bf16",
        gate="vector", window=64, alpha=0.5, seed=5, outlier_frac=0.01),
}

GATE_MODES = {"scalar": 0, "vector": 1}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("only finite values are rounded here")
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Return the canonical stored values as float32 (bf16-exact for bf16)."""
    x = np.asarray(x, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def prefill_inputs(B: int, T: int, H_q: int, H_kv: int, d: int, dtype: str,
                   seed: int, outlier_frac: float = 0.0, outlier_scale: float = 8.0,
                   **_ignored) -> dict:
    """q, k, v ~ N(0, 1), drawn in that order from PCG64(seed).

    With outlier_frac > 0, round(outlier_frac * B*T*H_kv) distinct (b, t, h_kv)
    key rows, chosen without replacement by the same generator after the
    q, k, v draws, are multiplied by `outlier_scale` (exact in bf16 for 8).
    Returned arrays are float32 holding the canonical stored values.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, H_q, d), dtype=np.float32)
    k = rng.standard_normal((B, T, H_kv, d), dtype=np.float32)
    v = rng.standard_normal((B, T, H_kv, d), dtype=np.float32)
    n_out = int(round(outlier_frac * B * T * H_kv))
    rows = np.zeros(0, dtype=np.int64)
    if n_out > 0:
        rows = rng.choice(B * T * H_kv, size=n_out, replace=False)
        kf = k.reshape(B * T * H_kv, d)
        kf[rows] *= np.float32(outlier_scale)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
                outlier_rows=np.sort(rows))


def grad_output(shape, dtype: str, seed: int, scale: float = 1.0) -> np.ndarray:
    """Upstream gradient dO ~ scale * N(0, 1) of the given shape, from
    PCG64(SeedSequence([seed, 7])), as canonical stored values."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return _store(np.float32(scale) * rng.standard_normal(tuple(shape), dtype=np.float32), dtype)


def config_prefill_inputs(name: str, T: int | None = None) -> dict:
    """Inputs of a named prefill workload (optionally only its first T tokens).

    A prefix is taken after drawing the full-length tensors, so its values are
    exactly the first T tokens of the full workload.
    """
    cfg = CONFIGS[name]
    assert cfg["kind"] == "prefill"
    x = prefill_inputs(**cfg)
    if T is not None and T < cfg["T"]:
        for key in ("q", "k", "v"):
            x[key] = np.ascontiguousarray(x[key][:, :T])
    return x


def decode_initial(N: int, H_kv: int, d: int, window: int, dtype: str, seed: int,
                   pos0: int, state_std: float = 0.1, **_ignored) -> dict:
    """Initial decode state: S ~ state_std*N(0,1) (fp32), ring k/v ~ N(0,1).

    Drawn from PCG64(seed) in the order S, ring_k, ring_v. Every sequence has
    consumed `pos0` tokens, so every ring slot holds a valid token when
    pos0 >= window.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S = (np.float32(state_std) *
         rng.standard_normal((N, H_kv, d, d), dtype=np.float32)).astype(np.float32)
    ring_k = rng.standard_normal((N, H_kv, window, d), dtype=np.float32)
    ring_v = rng.standard_normal((N, H_kv, window, d), dtype=np.float32)
    pos = np.full((N,), pos0, dtype=np.int64)
    return dict(S=S, ring_k=_store(ring_k, dtype), ring_v=_store(ring_v, dtype), pos=pos)


def decode_step_inputs(N: int, H_q: int, H_kv: int, d: int, dtype: str, seed: int,
                       step: int, **_ignored) -> dict:
    """Fresh q, k, v ~ N(0,1) for one decode step, from PCG64(SeedSequence([seed, step]))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, step])))
    q = rng.standard_normal((N, H_q, d), dtype=np.float32)
    k = rng.standard_normal((N, H_kv, d), dtype=np.float32)
    v = rng.standard_normal((N, H_kv, d), dtype=np.float32)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype))
