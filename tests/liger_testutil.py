"""Helpers shared by the GPU parity tests: moving seeded inputs to the GPU,
calling the library through its binding, and the parity bars.

Parity bars (max-norm, measured against the float64 oracle):
  fp32 path : ||gpu - ref||_inf <= 1e-4 * ||ref||_inf for o, the alpha = 1
              output and S_T.
  bf16 path : max |gpu - ref| <= 2e-2 on o (unit-scale outputs);
              the alpha = 1 output within 2e-2 * ||ref||_inf (the recurrent
              part alone is ~25x smaller than the window part, so it gets a
              relative bar of its own); S_T within 1e-2 * ||ref||_inf.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gated_linear_recurrent_amd as gla

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
CODE_DT = {"f32": gla.LIGER_F32, "bf16": gla.LIGER_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array holding storage-exact values -> device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(TORCH_DT[dtype]).contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_prefill(x: dict, dtype: str, gate: int, window: int, alpha: float, cps: int = 0, poison=True):
    q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan")) if poison else torch.empty_like(q)
    B, T, H_q, d = q.shape
    S_T = torch.full((B, k.shape[2], d, d), float("nan"), dtype=torch.float32, device=DEV)
    gla.liger_attn_prefill(q, k, v, gate, window, alpha, o=o, S_T=S_T, chunks_per_segment=cps)
    torch.cuda.synchronize()
    return o, S_T


def rel_inf(a, ref) -> float:
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-30))


def abs_inf(a, ref) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(ref, np.float64))))


def check_prefill(dtype: str, o_gpu, o_ref, S_gpu, S_ref, o1_gpu=None, o1_ref=None, tag=""):
    """Apply the parity bars; returns a dict of the measured errors."""
    o_gpu, S_gpu = np.asarray(o_gpu), np.asarray(S_gpu)
    assert np.all(np.isfinite(o_gpu)), f"{tag}: non-finite (unwritten?) outputs"
    assert np.all(np.isfinite(S_gpu)), f"{tag}: non-finite state"
    err = {}
    if dtype == "f32":
        err["o_rel"] = rel_inf(o_gpu, o_ref)
        err["S_rel"] = rel_inf(S_gpu, S_ref)
        assert err["o_rel"] <= 1e-4, (tag, err)
        assert err["S_rel"] <= 1e-4, (tag, err)
        if o1_gpu is not None:
            err["o1_rel"] = rel_inf(o1_gpu, o1_ref)
            assert err["o1_rel"] <= 1e-4, (tag, err)
    else:
        err["o_abs"] = abs_inf(o_gpu, o_ref)
        err["S_rel"] = rel_inf(S_gpu, S_ref)
        assert err["o_abs"] <= 2e-2, (tag, err)
        assert err["S_rel"] <= 1e-2, (tag, err)
        if o1_gpu is not None:
            err["o1_rel"] = rel_inf(o1_gpu, o1_ref)
            assert err["o1_rel"] <= 2e-2, (tag, err)
    say(f"  {tag}: {err}")
    return err
