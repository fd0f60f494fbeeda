"""Python binding of the Liger Attention C ABI (include/liger_attn.h).

Argument marshalling only: tensors become device pointers plus the current
HIP stream, and every computation runs in the HIP kernels of
libliger_attn.so. torch provides device memory and streams. There is no
fallback: if the library is missing or a call fails, a LigerError is raised.

The functions carry the C names:
  liger_attn_prefill, liger_attn_prefill_workspace_size,
  liger_attn_decode_step, liger_kv_ring_fill, liger_last_error
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libliger_attn.so")

LIGER_OK = 0
LIGER_E_INVALID_ARG = -1
LIGER_E_UNSUPPORTED = -2
LIGER_E_HIP = -3
LIGER_E_WORKSPACE = -4
STATUS_NAMES = {0: "LIGER_OK", -1: "LIGER_E_INVALID_ARG", -2: "LIGER_E_UNSUPPORTED",
                -3: "LIGER_E_HIP", -4: "LIGER_E_WORKSPACE"}

LIGER_GATE_SCALAR_MEAN = 0
LIGER_GATE_VECTOR_AVGPOOL4 = 1
LIGER_F32 = 0
LIGER_BF16 = 1
LIGER_STAGE_SEGMENT_STATES = 1
LIGER_STAGE_CARRY_SCAN = 2
LIGER_STAGE_OUTPUT = 4

# Every symbol the header declares (checked by the CPU tests).
EXPORTED = (
    "liger_attn_prefill_workspace_size",
    "liger_attn_prefill_workspace_size_ex",
    "liger_attn_prefill",
    "liger_attn_prefill_ex",
    "liger_attn_prefill_stages",
    "liger_attn_prefill_noalloc",
    "liger_attn_prefill_noalloc_max_workspace",
    "liger_attn_prefill_continue",
    "liger_attn_decode_step",
    "liger_kv_ring_fill",
    "liger_attn_full_causal",
    "liger_attn_prefill_sinks",
    "liger_attn_prefill_continue_sinks",
    "liger_attn_decode_step_sinks",
    "liger_attn_prefill_backward_workspace_size",
    "liger_attn_prefill_backward",
    "liger_last_error",
)


class LigerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class liger_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H_q", ctypes.c_int32),
                ("H_kv", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class liger_kv_ring(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("sync", ctypes.c_void_p), ("window", ctypes.c_int32)]


class liger_sinks(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libliger_attn.so (built by gated_linear_recurrent_amd.build_lib)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LigerError(LIGER_E_HIP, f"{path} is not built; run python -m gated_linear_recurrent_amd.build_lib")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    shp = ctypes.POINTER(liger_shape)
    ring = ctypes.POINTER(liger_kv_ring)
    lib.liger_attn_prefill_workspace_size.argtypes = [shp]
    lib.liger_attn_prefill_workspace_size.restype = sz
    lib.liger_attn_prefill_workspace_size_ex.argtypes = [shp, i32]
    lib.liger_attn_prefill_workspace_size_ex.restype = sz
    lib.liger_attn_prefill.argtypes = [vp, vp, vp, i32, i32, f32, shp, vp, vp, vp, sz, vp]
    lib.liger_attn_prefill.restype = i32
    lib.liger_attn_prefill_ex.argtypes = [vp, vp, vp, i32, i32, f32, shp, vp, vp, vp, sz, i32, vp]
    lib.liger_attn_prefill_ex.restype = i32
    lib.liger_attn_prefill_stages.argtypes = [vp, vp, vp, i32, i32, f32, shp, vp, vp, vp, sz, i32, i32, vp]
    lib.liger_attn_prefill_stages.restype = i32
    lib.liger_attn_prefill_noalloc.argtypes = [vp, vp, vp, i32, i32, f32, shp, vp, vp, vp]
    lib.liger_attn_prefill_noalloc.restype = i32
    lib.liger_attn_prefill_noalloc_max_workspace.argtypes = []
    lib.liger_attn_prefill_noalloc_max_workspace.restype = sz
    lib.liger_attn_prefill_continue.argtypes = [vp, vp, vp, vp, ring, i32, f32, shp, vp, vp, vp, sz, vp]
    lib.liger_attn_prefill_continue.restype = i32
    lib.liger_attn_decode_step.argtypes = [vp, vp, vp, vp, ring, i32, f32, shp, vp, vp]
    lib.liger_attn_decode_step.restype = i32
    lib.liger_kv_ring_fill.argtypes = [vp, vp, shp, ring, vp]
    lib.liger_kv_ring_fill.restype = i32
    lib.liger_attn_full_causal.argtypes = [vp, vp, vp, shp, vp, vp]
    lib.liger_attn_full_causal.restype = i32
    snk = ctypes.POINTER(liger_sinks)
    lib.liger_attn_prefill_sinks.argtypes = [vp, vp, vp, snk, i32, i32, f32, shp, vp, vp, vp, sz, vp]
    lib.liger_attn_prefill_sinks.restype = i32
    lib.liger_attn_prefill_continue_sinks.argtypes = [vp, vp, vp, vp, ring, snk, i32, f32, shp, vp, vp, vp, sz, vp]
    lib.liger_attn_prefill_continue_sinks.restype = i32
    lib.liger_attn_decode_step_sinks.argtypes = [vp, vp, vp, vp, ring, snk, i32, f32, shp, vp, vp]
    lib.liger_attn_decode_step_sinks.restype = i32
    lib.liger_attn_prefill_backward_workspace_size.argtypes = [shp]
    lib.liger_attn_prefill_backward_workspace_size.restype = sz
    lib.liger_attn_prefill_backward.argtypes = [vp, vp, vp, vp, i32, i32, f32, shp, vp, vp, vp, vp, sz, vp]
    lib.liger_attn_prefill_backward.restype = i32
    lib.liger_last_error.argtypes = []
    lib.liger_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def liger_last_error() -> str:
    return load_library().liger_last_error().decode()


def _check(status: int) -> None:
    if status != LIGER_OK:
        raise LigerError(status, liger_last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LIGER_BF16
    if t.dtype == torch.float32:
        return LIGER_F32
    raise LigerError(LIGER_E_INVALID_ARG, f"unsupported dtype {t.dtype}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise LigerError(LIGER_E_INVALID_ARG, "tensors must live in GPU memory")
    if not t.is_contiguous():
        raise LigerError(LIGER_E_INVALID_ARG, "tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_shape(B: int, T: int, H_q: int, H_kv: int, d: int, dtype: int) -> liger_shape:
    return liger_shape(B, T, H_q, H_kv, d, dtype)


def liger_attn_prefill_workspace_size(B: int, T: int, H_q: int, H_kv: int, d: int, dtype: int,
                                      chunks_per_segment: int = 0) -> int:
    shp = make_shape(B, T, H_q, H_kv, d, dtype)
    return int(load_library().liger_attn_prefill_workspace_size_ex(ctypes.byref(shp), chunks_per_segment))


def liger_attn_prefill_backward_workspace_size(B: int, T: int, H_q: int, H_kv: int, d: int) -> int:
    shp = make_shape(B, T, H_q, H_kv, d, LIGER_BF16)
    return int(load_library().liger_attn_prefill_backward_workspace_size(ctypes.byref(shp)))


def _sinks_c(sinks):
    """(sink_k, sink_v) device tensors [H_kv, n, d] -> liger_sinks."""
    sk, sv = sinks
    return liger_sinks(_ptr(sk), _ptr(sv), int(sk.shape[1]))


def liger_attn_prefill(q, k, v, gate_mode: int, window: int, alpha: float, *, o=None, S_T=None,
                       workspace=None, chunks_per_segment: int = 0, stage_mask: int = 7, stream=None,
                       sinks=None):
    """Prefill from a zero state. q [B,T,H_q,d], k/v [B,T,H_kv,d] -> (o, S_T fp32 [B,H_kv,d,d]).

    stage_mask < 7 enqueues only some kernels (liger_attn_prefill_stages).
    sinks = (sink_k, sink_v) [H_kv, n, d] prepends meta-memory tokens to every
    window (liger_attn_prefill_sinks)."""
    torch = _torch()
    lib = load_library()
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    shp = make_shape(B, T, H_q, H_kv, d, _dtype_code(q))
    if o is None:
        o = torch.empty_like(q)
    if S_T is None:
        S_T = torch.empty((B, H_kv, d, d), dtype=torch.float32, device=q.device)
    need = int(lib.liger_attn_prefill_workspace_size_ex(ctypes.byref(shp), chunks_per_segment))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if sinks is not None:
        if stage_mask != 7 or chunks_per_segment != 0:
            raise LigerError(LIGER_E_INVALID_ARG, "sinks take the default stages and segment plan")
        cs = _sinks_c(sinks)
        _check(lib.liger_attn_prefill_sinks(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), gate_mode, window, alpha,
                                            ctypes.byref(shp), _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes,
                                            _stream(stream)))
        return o, S_T
    _check(lib.liger_attn_prefill_stages(_ptr(q), _ptr(k), _ptr(v), gate_mode, window, alpha,
                                         ctypes.byref(shp), _ptr(o), _ptr(S_T), _ptr(workspace),
                                         ws_bytes, chunks_per_segment, stage_mask, _stream(stream)))
    return o, S_T


def liger_attn_prefill_noalloc(q, k, v, gate_mode: int, window: int, alpha: float, *, o, S_T, stream=None):
    """liger_attn_prefill with the workspace in the library's static scratch
    (no device allocation by the library). o and S_T are caller buffers."""
    lib = load_library()
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    shp = make_shape(B, T, H_q, H_kv, d, _dtype_code(q))
    _check(lib.liger_attn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), gate_mode, window, alpha, ctypes.byref(shp),
                                          _ptr(o), _ptr(S_T), _stream(stream)))
    return o, S_T


def liger_attn_prefill_noalloc_max_workspace() -> int:
    return int(load_library().liger_attn_prefill_noalloc_max_workspace())


@dataclass
class KVRing:
    """Device buffers of the sliding-window KV ring (see liger_kv_ring)."""
    k: object     # [N, H_kv, window, d]
    v: object
    pos: object   # [N] int64
    sync: object  # [N] int32 (uint32 counters), zero between calls
    window: int

    @classmethod
    def empty(cls, N: int, H_kv: int, window: int, d: int, dtype, device):
        torch = _torch()
        return cls(torch.zeros((N, H_kv, window, d), dtype=dtype, device=device),
                   torch.zeros((N, H_kv, window, d), dtype=dtype, device=device),
                   torch.zeros((N,), dtype=torch.int64, device=device),
                   torch.zeros((N,), dtype=torch.int32, device=device), window)

    def as_c(self) -> liger_kv_ring:
        return liger_kv_ring(_ptr(self.k), _ptr(self.v), _ptr(self.pos), _ptr(self.sync), self.window)


def liger_kv_ring_fill(k, v, ring: KVRing, stream=None) -> KVRing:
    """Ring after a prompt k/v [B,T,H_kv,d]: last min(T, window) tokens at slot t mod window."""
    lib = load_library()
    B, T, H_kv, d = k.shape
    shp = make_shape(B, T, H_kv, H_kv, d, _dtype_code(k))
    cring = ring.as_c()
    _check(lib.liger_kv_ring_fill(_ptr(k), _ptr(v), ctypes.byref(shp), ctypes.byref(cring), _stream(stream)))
    return ring


def liger_attn_prefill_continue(q, k, v, S0, ring: KVRing, gate_mode: int, alpha: float, *, o=None, S_T=None,
                                workspace=None, stream=None, sinks=None):
    """T more tokens after ring.pos[b] consumed ones, from state S0 (not modified) and the ring
    (updated in place: last tokens written, pos += T). Window = ring.window. -> (o, S_T)."""
    torch = _torch()
    lib = load_library()
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    shp = make_shape(B, T, H_q, H_kv, d, _dtype_code(q))
    if o is None:
        o = torch.empty_like(q)
    if S_T is None:
        S_T = torch.empty((B, H_kv, d, d), dtype=torch.float32, device=q.device)
    need = int(lib.liger_attn_prefill_workspace_size_ex(ctypes.byref(shp), 0))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cring = ring.as_c()
    if sinks is not None:
        cs = _sinks_c(sinks)
        _check(lib.liger_attn_prefill_continue_sinks(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), ctypes.byref(cring),
                                                     ctypes.byref(cs), gate_mode, alpha, ctypes.byref(shp), _ptr(o),
                                                     _ptr(S_T), _ptr(workspace), ws_bytes, _stream(stream)))
        return o, S_T
    _check(lib.liger_attn_prefill_continue(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), ctypes.byref(cring), gate_mode,
                                           alpha, ctypes.byref(shp), _ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes,
                                           _stream(stream)))
    return o, S_T


def liger_attn_full_causal(q, k, v, *, o=None, stream=None):
    """The hybrid's softmax layer: q [B,T,H_q,d], k/v [B,T,H_kv,d] (bf16); returns o."""
    torch = _torch()
    lib = load_library()
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    shp = make_shape(B, T, H_q, H_kv, d, _dtype_code(q))
    if o is None:
        o = torch.empty_like(q)
    _check(lib.liger_attn_full_causal(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(shp), _ptr(o), _stream(stream)))
    return o


def liger_attn_prefill_backward(q, k, v, dO, gate_mode: int, window: int, alpha: float, *, dq=None, dk=None,
                                dv=None, workspace=None, stream=None):
    """Gradients of sum(o * dO) for o = liger_attn_prefill(q, k, v, ...): q, dO [B,T,H_q,d], k/v [B,T,H_kv,d]
    (bf16); returns float32 (dq, dk, dv)."""
    torch = _torch()
    lib = load_library()
    B, T, H_q, d = q.shape
    H_kv = k.shape[2]
    shp = make_shape(B, T, H_q, H_kv, d, _dtype_code(q))
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    need = lib.liger_attn_prefill_backward_workspace_size(ctypes.byref(shp))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.liger_attn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), gate_mode, window, alpha,
                                           ctypes.byref(shp), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                           ws_bytes, _stream(stream)))
    return dq, dk, dv


def liger_attn_decode_step(q, k, v, S, ring: KVRing, gate_mode: int, alpha: float, *, o=None, stream=None,
                           sinks=None):
    """One token per sequence: q [N,H_q,d], k/v [N,H_kv,d]; S and ring updated in place; returns o."""
    torch = _torch()
    lib = load_library()
    N, H_q, d = q.shape
    H_kv = k.shape[1]
    shp = make_shape(N, 1, H_q, H_kv, d, _dtype_code(q))
    if o is None:
        o = torch.empty_like(q)
    cring = ring.as_c()
    if sinks is not None:
        cs = _sinks_c(sinks)
        _check(lib.liger_attn_decode_step_sinks(_ptr(q), _ptr(k), _ptr(v), _ptr(S), ctypes.byref(cring),
                                                ctypes.byref(cs), gate_mode, alpha, ctypes.byref(shp), _ptr(o),
                                                _stream(stream)))
        return o
    _check(lib.liger_attn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), ctypes.byref(cring), gate_mode,
                                      alpha, ctypes.byref(shp), _ptr(o), _stream(stream)))
    return o
