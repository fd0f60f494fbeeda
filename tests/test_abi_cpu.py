"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects invalid arguments before making any HIP call.

No kernel runs here. Pointers handed to the library are fake but 16-byte
aligned; every call below fails validation, so they are never dereferenced.
The one call that passes validation (no-GPU error path) runs only where no
GPU is visible.
"""
import ctypes
import os
import re

import pytest

import gated_linear_recurrent_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # aligned, never dereferenced
G = 1 << 32     # spacing of fake buffers whose byte ranges must not overlap


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.LIB_PATH):
        from gated_linear_recurrent_amd import build_lib
        build_lib.build()
    return gla.load_library()


def _header_functions():
    with open(os.path.join(ROOT, "include", "liger_attn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|size_t|liger_status)\s+(liger_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    declared = _header_functions()
    assert set(declared) == set(gla.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_exports_are_plain_c_symbols():
    out = os.popen(f"nm -D --defined-only {gla.LIB_PATH}").read()
    for name in gla.EXPORTED:
        assert re.search(rf"\bT {name}$", out, re.M), name


def _shape(**kw):
    base = dict(B=1, T=128, H_q=4, H_kv=1, d=128, dtype=gla.LIGER_BF16)
    base.update(kw)
    return gla.liger_shape(**base)


def _prefill(lib, shape, gate=1, window=64, alpha=0.5, q=FAKE, k=FAKE, v=FAKE, o=FAKE + G,
             S=FAKE + 2 * G, ws=None, ws_bytes=0, cps=0):
    return lib.liger_attn_prefill_ex(q, k, v, gate, window, alpha, ctypes.byref(shape), o, S, ws,
                                     ws_bytes, cps, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), gla.LIGER_E_INVALID_ARG),
    (dict(T=0), gla.LIGER_E_INVALID_ARG),
    (dict(H_kv=0), gla.LIGER_E_INVALID_ARG),
    (dict(H_q=6, H_kv=4), gla.LIGER_E_INVALID_ARG),
    (dict(d=96), gla.LIGER_E_UNSUPPORTED),
    (dict(d=256), gla.LIGER_E_UNSUPPORTED),
    (dict(dtype=7), gla.LIGER_E_INVALID_ARG),
])
def test_prefill_rejects_bad_shapes(lib, kw, code):
    assert _prefill(lib, _shape(**kw)) == code
    assert gla.liger_last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(gate=2), gla.LIGER_E_INVALID_ARG),
    (dict(window=0), gla.LIGER_E_INVALID_ARG),
    (dict(window=65), gla.LIGER_E_INVALID_ARG),
    (dict(alpha=-0.1), gla.LIGER_E_INVALID_ARG),
    (dict(alpha=1.5), gla.LIGER_E_INVALID_ARG),
    (dict(alpha=float("nan")), gla.LIGER_E_INVALID_ARG),
    (dict(q=None), gla.LIGER_E_INVALID_ARG),
    (dict(k=FAKE + 8), gla.LIGER_E_INVALID_ARG),
    (dict(o=FAKE), gla.LIGER_E_INVALID_ARG),      # aliases q
    (dict(o=FAKE + 4096), gla.LIGER_E_INVALID_ARG),  # starts inside q
    (dict(S=FAKE + G + 4096), gla.LIGER_E_INVALID_ARG),  # S_T starts inside o
    (dict(S=FAKE + 256), gla.LIGER_E_INVALID_ARG),  # S_T starts inside q
    (dict(S=None), gla.LIGER_E_INVALID_ARG),
    (dict(cps=-1), gla.LIGER_E_INVALID_ARG),
])
def test_prefill_rejects_bad_arguments(lib, kw, code):
    assert _prefill(lib, _shape(T=4096), **kw) == code


def test_prefill_workspace_checks(lib):
    shp = _shape(T=8192, H_q=32, H_kv=8)
    need = lib.liger_attn_prefill_workspace_size(ctypes.byref(shp))
    assert need > 0 and need % 16 == 0
    assert _prefill(lib, shp, ws=None) == gla.LIGER_E_WORKSPACE
    assert _prefill(lib, shp, ws=FAKE + 1 << 20, ws_bytes=need - 1) == gla.LIGER_E_WORKSPACE
    assert _prefill(lib, shp, ws=(FAKE + 1 << 20) + 4, ws_bytes=need) == gla.LIGER_E_INVALID_ARG


def test_adjacent_buffers_are_accepted(lib):
    """Byte ranges that touch without sharing a byte pass the overlap checks
    (the call then stops at the missing workspace)."""
    shp = _shape(T=64)
    qbytes = 64 * 4 * 128 * 2
    assert _prefill(lib, shp, o=FAKE + qbytes, S=FAKE + 2 * qbytes) == gla.LIGER_E_WORKSPACE
    assert _prefill(lib, shp, o=FAKE + qbytes - 16, S=FAKE + 2 * qbytes) == gla.LIGER_E_INVALID_ARG


def test_workspace_size_formula(lib):
    # carries of every segment but the last, (d*d + d) fp32 per (b, kv head,
    # segment), then one d*d fp32 running-state slot per (b, kv head, segment)
    for T, cps in [(64, 1), (65, 1), (8192, 4), (1000, 3)]:
        shp = _shape(B=2, T=T, H_q=8, H_kv=2)
        n_chunks = -(-T // 64)
        size = lib.liger_attn_prefill_workspace_size_ex(ctypes.byref(shp), cps)
        n_seg = -(-n_chunks // min(cps, n_chunks))
        assert size == 2 * 2 * ((n_seg - 1) * (128 * 128 + 128) + n_seg * 128 * 128) * 4
    size0 = lib.liger_attn_prefill_workspace_size(ctypes.byref(_shape(T=8192, H_q=32, H_kv=8)))
    assert size0 > 0 and size0 % 16 == 0
    # fp32 at d = 128: a state-operand slot beside each running-state slot,
    # and 64 halo K and V rows per (b, kv head)
    for T, cps in [(64, 1), (65, 1), (1000, 3)]:
        shp = _shape(B=2, T=T, H_q=8, H_kv=2, dtype=gla.LIGER_F32)
        n_chunks = -(-T // 64)
        size = lib.liger_attn_prefill_workspace_size_ex(ctypes.byref(shp), cps)
        n_seg = -(-n_chunks // min(cps, n_chunks))
        assert size == 2 * 2 * ((n_seg - 1) * (128 * 128 + 128) + 2 * n_seg * 128 * 128 + 2 * 64 * 128) * 4
    assert lib.liger_attn_prefill_workspace_size(ctypes.byref(_shape(d=96))) == 0
    assert lib.liger_attn_prefill_workspace_size(None) == 0


def _ring(window=64, k=FAKE + 8 * G, v=FAKE + 9 * G, pos=FAKE + 10 * G, sync=FAKE + 11 * G):
    return gla.liger_kv_ring(k, v, pos, sync, window)


def _decode(lib, shape, ring, gate=1, alpha=0.5, q=FAKE + 12 * G, k=FAKE + 13 * G, v=FAKE + 14 * G,
            S=FAKE + 15 * G, o=FAKE + 16 * G):
    return lib.liger_attn_decode_step(q, k, v, S, ctypes.byref(ring) if ring is not None else None,
                                      gate, alpha, ctypes.byref(shape), o, None)


@pytest.mark.parametrize("kw,rkw,code", [
    (dict(), dict(window=0), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(window=65), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(pos=None), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(sync=None), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(k=FAKE + 2), gla.LIGER_E_INVALID_ARG),
    (dict(H_q=12, H_kv=1), dict(), gla.LIGER_E_UNSUPPORTED),
    (dict(d=32), dict(), gla.LIGER_E_UNSUPPORTED),
    (dict(B=0), dict(), gla.LIGER_E_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(lib, kw, rkw, code):
    assert _decode(lib, _shape(**kw), _ring(**rkw)) == code


def test_decode_rejects_null_ring_and_alias(lib):
    assert _decode(lib, _shape(), None) == gla.LIGER_E_INVALID_ARG
    assert _decode(lib, _shape(), _ring(), o=FAKE + 12 * G) == gla.LIGER_E_INVALID_ARG
    assert _decode(lib, _shape(), _ring(), gate=-1) == gla.LIGER_E_INVALID_ARG


# decode writes o, S and the ring (k, v, pos, sync): each must be disjoint from
# the inputs and from the others (shape: N = 1, H_q = 4, H_kv = 1, d = 128, bf16,
# window 64: S 64 KiB, ring k and v 16 KiB each, pos 8 B, sync 4 B)
@pytest.mark.parametrize("dkw,rkw,msg", [
    (dict(S=FAKE + 12 * G + 512), {}, "S must not overlap q"),
    (dict(S=FAKE + 16 * G - 4096), {}, "o must not overlap S"),
    ({}, dict(k=FAKE + 13 * G), "kv_ring->k must not overlap k"),
    ({}, dict(v=FAKE + 14 * G + 128), "kv_ring->v must not overlap v"),
    ({}, dict(v=FAKE + 8 * G + 16384 - 16), "kv_ring->k must not overlap kv_ring->v"),
    ({}, dict(pos=FAKE + 15 * G + 64), "S must not overlap kv_ring->pos"),
    ({}, dict(sync=FAKE + 10 * G), "kv_ring->pos must not overlap kv_ring->sync"),
    ({}, dict(sync=FAKE + 9 * G + 16), "kv_ring->v must not overlap kv_ring->sync"),
    ({}, dict(pos=FAKE + 16 * G), "o must not overlap kv_ring->pos"),
])
def test_decode_rejects_overlapping_state(lib, dkw, rkw, msg):
    assert _decode(lib, _shape(), _ring(**rkw), **dkw) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == msg


def test_decode_state_buffers_may_touch(lib):
    """Buffers that touch without sharing a byte pass the overlap checks."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake pointers of this test must not reach a kernel")
    r = _ring(k=FAKE + 8 * G, v=FAKE + 8 * G + 16384, pos=FAKE + 8 * G + 32768, sync=FAKE + 8 * G + 32768 + 16)
    assert _decode(lib, _shape(), r) == gla.LIGER_E_HIP, gla.liger_last_error()


def _continue(lib, shape, ring, S0=FAKE + 3 * G, S_T=FAKE + 4 * G, o=FAKE + 5 * G, gate=1, alpha=0.5,
              ws=FAKE << 8, ws_bytes=1 << 40):
    return lib.liger_attn_prefill_continue(FAKE, FAKE + G, FAKE + 2 * G, S0,
                                           ctypes.byref(ring) if ring is not None else None, gate, alpha,
                                           ctypes.byref(shape), o, S_T, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,rkw,ckw,code", [
    (dict(), dict(), dict(S0=None), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(window=0), dict(), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(window=65), dict(), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(pos=None), dict(), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(sync=None), dict(), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(), dict(S_T=FAKE + 3 * G + 16), gla.LIGER_E_INVALID_ARG),    # S_T overlaps S0
    (dict(), dict(), dict(o=FAKE), gla.LIGER_E_INVALID_ARG),                   # o aliases q
    (dict(), dict(), dict(o=FAKE + 2 * G + 64), gla.LIGER_E_INVALID_ARG),      # o starts inside v
    (dict(), dict(), dict(S_T=FAKE + 5 * G + 512), gla.LIGER_E_INVALID_ARG),   # S_T starts inside o
    (dict(), dict(), dict(ws=None), gla.LIGER_E_WORKSPACE),
    (dict(T=0), dict(), dict(), gla.LIGER_E_INVALID_ARG),
    (dict(), dict(), dict(gate=5), gla.LIGER_E_INVALID_ARG),
])
def test_continue_rejects_bad_arguments(lib, kw, rkw, ckw, code):
    shp = _shape(**{**dict(T=256, H_q=4, H_kv=1), **kw})
    assert _continue(lib, shp, _ring(**rkw), **ckw) == code
    assert gla.liger_last_error() != ""


def test_continue_rejects_null_ring(lib):
    assert _continue(lib, _shape(T=256), None) == gla.LIGER_E_INVALID_ARG


@pytest.mark.parametrize("rkw,msg", [
    (dict(k=FAKE + 256), "kv_ring->k must not overlap k"),
    (dict(v=FAKE + G + 1024), "kv_ring->v must not overlap v"),
    (dict(pos=FAKE + 8 * G + 64), "kv_ring->k must not overlap kv_ring->pos"),
    (dict(sync=FAKE + 10 * G + 4), "kv_ring->pos must not overlap kv_ring->sync"),
])
def test_ring_fill_rejects_overlaps(lib, rkw, msg):
    shp = _shape()
    r = _ring(**rkw)
    assert lib.liger_kv_ring_fill(FAKE, FAKE + G, ctypes.byref(shp), ctypes.byref(r), None) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == msg


@pytest.mark.parametrize("rkw,ckw,msg", [
    (dict(k=FAKE + 5 * G), {}, "o must not overlap kv_ring->k"),
    (dict(pos=FAKE + 3 * G + 8), {}, "kv_ring->pos must not overlap S0"),
    ({}, dict(ws=FAKE + 64, ws_bytes=1 << 40), "workspace must not overlap q"),
    ({}, dict(ws=FAKE + 4 * G - 1024, ws_bytes=1 << 40), "workspace must not overlap S_T"),
])
def test_continue_rejects_overlaps(lib, rkw, ckw, msg):
    shp = _shape(T=256, H_q=4, H_kv=1)
    assert _continue(lib, shp, _ring(**rkw), **ckw) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == msg


def test_prefill_rejects_workspace_overlap(lib):
    shp = _shape(T=4096)
    need = lib.liger_attn_prefill_workspace_size(ctypes.byref(shp))
    assert _prefill(lib, shp, ws=FAKE + G - 4096, ws_bytes=need) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == "workspace must not overlap o"
    assert _prefill(lib, shp, ws=FAKE + 2 * G + 1024, ws_bytes=need) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == "workspace must not overlap S_T"
    assert _prefill(lib, shp, ws=FAKE + 4096, ws_bytes=need) == gla.LIGER_E_INVALID_ARG
    assert gla.liger_last_error() == "workspace must not overlap q"


def test_ring_fill_rejects_bad_arguments(lib):
    shp = _shape()
    assert lib.liger_kv_ring_fill(FAKE, FAKE, ctypes.byref(shp), None, None) == gla.LIGER_E_INVALID_ARG
    r = _ring(window=100)
    assert lib.liger_kv_ring_fill(FAKE, FAKE, ctypes.byref(shp), ctypes.byref(r), None) == gla.LIGER_E_INVALID_ARG
    r = _ring()
    assert lib.liger_kv_ring_fill(None, FAKE, ctypes.byref(shp), ctypes.byref(r), None) == gla.LIGER_E_INVALID_ARG


def test_no_gpu_returns_hip_error_instead_of_aborting(lib):
    """A valid call on a machine without a GPU fails with LIGER_E_HIP."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake pointers of this test must not reach a kernel")
    shp = _shape(T=64)
    need = lib.liger_attn_prefill_workspace_size(ctypes.byref(shp))
    st = _prefill(lib, shp, ws=FAKE << 8, ws_bytes=need)
    assert st == gla.LIGER_E_HIP, gla.liger_last_error()
    assert "launch" in gla.liger_last_error()


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(gla.LigerError):
        gla.liger_attn_prefill(q, k, k, 1, 64, 0.5, o=q.clone(), S_T=torch.zeros(1, 1, 128, 128),
                               workspace=None)


@pytest.mark.parametrize("kw,ptrs,code", [
    (dict(dtype=gla.LIGER_F32), {}, gla.LIGER_E_UNSUPPORTED),
    (dict(H_q=3, H_kv=1), {}, gla.LIGER_E_UNSUPPORTED),
    (dict(H_q=6, H_kv=4), {}, gla.LIGER_E_INVALID_ARG),
    (dict(d=96), {}, gla.LIGER_E_UNSUPPORTED),
    (dict(T=0), {}, gla.LIGER_E_INVALID_ARG),
    ({}, dict(q=None), gla.LIGER_E_INVALID_ARG),
    ({}, dict(v=FAKE + 2), gla.LIGER_E_INVALID_ARG),
    ({}, dict(o=FAKE), gla.LIGER_E_INVALID_ARG),
    ({}, dict(o=FAKE + G + 1024), gla.LIGER_E_INVALID_ARG),  # starts inside k
    ({}, dict(o=FAKE - 1024), gla.LIGER_E_INVALID_ARG),      # ends inside q
])
def test_full_causal_rejects_bad_arguments(lib, kw, ptrs, code):
    p = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, o=FAKE + 3 * G)
    p.update(ptrs)
    st = lib.liger_attn_full_causal(p["q"], p["k"], p["v"], ctypes.byref(_shape(**kw)), p["o"], None)
    assert st == code, gla.liger_last_error()


@pytest.mark.parametrize("n,k,v,code", [
    (0, FAKE, FAKE, gla.LIGER_E_INVALID_ARG),
    (17, FAKE, FAKE, gla.LIGER_E_INVALID_ARG),
    (4, None, FAKE, gla.LIGER_E_INVALID_ARG),
    (4, FAKE, FAKE + 8, gla.LIGER_E_INVALID_ARG),
])
def test_sinks_rejected(lib, n, k, v, code):
    sk = gla.liger_sinks(k, v, n)
    shp = _shape()
    st = lib.liger_attn_prefill_sinks(FAKE, FAKE, FAKE, ctypes.byref(sk), 1, 64, 0.5, ctypes.byref(shp),
                                      FAKE + 4096, FAKE + 8192, FAKE << 8, 1 << 30, None)
    assert st == code, gla.liger_last_error()
    ring = gla.liger_kv_ring(FAKE, FAKE, FAKE, FAKE, 64)
    st = lib.liger_attn_decode_step_sinks(FAKE, FAKE, FAKE, FAKE, ctypes.byref(ring), ctypes.byref(sk), 1, 0.5,
                                          ctypes.byref(shp), FAKE + 4096, None)
    assert st == code, gla.liger_last_error()
    st = lib.liger_attn_prefill_continue_sinks(FAKE, FAKE, FAKE, FAKE, ctypes.byref(ring), ctypes.byref(sk), 1, 0.5,
                                               ctypes.byref(shp), FAKE + 4096, FAKE + 8192, FAKE << 8, 1 << 30, None)
    assert st == code, gla.liger_last_error()


def test_sinks_null_struct_rejected(lib):
    shp = _shape()
    st = lib.liger_attn_prefill_sinks(FAKE, FAKE, FAKE, None, 1, 64, 0.5, ctypes.byref(shp),
                                      FAKE + 4096, FAKE + 8192, FAKE << 8, 1 << 30, None)
    assert st == gla.LIGER_E_INVALID_ARG
    assert "sinks" in gla.liger_last_error()


@pytest.mark.parametrize("kw,ptrs,extra,code", [
    (dict(dtype=gla.LIGER_F32, d=64), {}, {}, gla.LIGER_E_UNSUPPORTED),
    (dict(d=96), {}, {}, gla.LIGER_E_UNSUPPORTED),
    ({}, {}, dict(window=0), gla.LIGER_E_INVALID_ARG),
    ({}, {}, dict(window=65), gla.LIGER_E_INVALID_ARG),
    ({}, {}, dict(alpha=1.5), gla.LIGER_E_INVALID_ARG),
    ({}, {}, dict(gate=2), gla.LIGER_E_INVALID_ARG),
    ({}, dict(dO=None), {}, gla.LIGER_E_INVALID_ARG),
    ({}, dict(dq=FAKE), {}, gla.LIGER_E_INVALID_ARG),
    ({}, dict(dq=FAKE + 4096), {}, gla.LIGER_E_INVALID_ARG),       # starts inside q
    ({}, dict(dv=FAKE + 4 * G), {}, gla.LIGER_E_INVALID_ARG),      # same as dq
    ({}, dict(dk=FAKE + 4 * G + 2048), {}, gla.LIGER_E_INVALID_ARG),  # starts inside dq
    ({}, dict(dk=FAKE + 5 * G + 8), {}, gla.LIGER_E_INVALID_ARG),  # misaligned
    ({}, {}, dict(ws_bytes=16), gla.LIGER_E_WORKSPACE),
    ({}, dict(dv=(FAKE << 8) + 4096), {}, gla.LIGER_E_INVALID_ARG),  # inside the workspace
])
def test_backward_rejects_bad_arguments(lib, kw, ptrs, extra, code):
    p = dict(q=FAKE, k=FAKE + G, v=FAKE + 2 * G, dO=FAKE + 3 * G, dq=FAKE + 4 * G, dk=FAKE + 5 * G,
             dv=FAKE + 6 * G)
    p.update(ptrs)
    e = dict(gate=1, window=64, alpha=0.5, ws_bytes=1 << 40)
    e.update(extra)
    shp = _shape(**kw)
    st = lib.liger_attn_prefill_backward(p["q"], p["k"], p["v"], p["dO"], e["gate"], e["window"], e["alpha"],
                                         ctypes.byref(shp), p["dq"], p["dk"], p["dv"], FAKE << 8, e["ws_bytes"],
                                         None)
    assert st == code, gla.liger_last_error()


def test_backward_workspace_size(lib):
    """Two record sets of d*d + d floats per chunk boundary, per-row gate
    gradients, chunk sums and two window statistics per query row."""
    shp = _shape(B=2, T=130, H_q=8, H_kv=2, d=64)
    n = 3
    want = 4 * (2 * 2 * 2 * (n - 1) * (64 * 64 + 64) + 2 * 2 * 130 * 64 + 2 * 2 * n * 64 + 2 * 130 * 8 * 2)
    assert lib.liger_attn_prefill_backward_workspace_size(ctypes.byref(shp)) == want
    assert lib.liger_attn_prefill_backward_workspace_size(ctypes.byref(_shape(T=0))) == 0


def test_noalloc_limit_and_rejection(lib):
    """The allocation-free prefill states its scratch size and refuses larger
    shapes (and invalid ones) before any HIP call."""
    assert lib.liger_attn_prefill_noalloc_max_workspace() == 32 << 20
    big = _shape(B=65, T=64, H_q=32, H_kv=8)
    assert lib.liger_attn_prefill_workspace_size(ctypes.byref(big)) > 32 << 20
    st = lib.liger_attn_prefill_noalloc(FAKE, FAKE + G, FAKE + 2 * G, 0, 64, 0.5, ctypes.byref(big),
                                        FAKE + 3 * G, FAKE + 4 * G, None)
    assert st == gla.LIGER_E_WORKSPACE and "32 MiB" not in gla.liger_last_error()
    assert str(32 << 20) in gla.liger_last_error()
    st = lib.liger_attn_prefill_noalloc(FAKE, FAKE, FAKE, 0, 64, 0.5, ctypes.byref(_shape()), FAKE, FAKE + G, None)
    assert st == gla.LIGER_E_INVALID_ARG  # o aliases q
    st = lib.liger_attn_prefill_noalloc(FAKE, FAKE, FAKE, 0, 0, 0.5, ctypes.byref(_shape()), FAKE + G, FAKE + 2 * G,
                                        None)
    assert st == gla.LIGER_E_INVALID_ARG  # window 0
