"""HIP-graph replays of the library's launches against the same launches run
eagerly: a captured run of decode steps (state, ring, pos and the arrival
counters all round-trip through memory) and a captured prefill. Each graph is
replayed several times with the program's own eager work (state resets,
output poisoning) and synchronisations between the replays; every replay
must reproduce the eager results bit for bit (same kernels, same inputs).
"""
import pytest
import torch

import gated_linear_recurrent_amd as gla
from liger_testutil import DEV, say
from synth import prefill_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            fn()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("gate", [0, 1])
def test_decode_steps_replayed_from_a_graph(gate):
    N, H_kv, n_rep, d, T0, steps, window = 4, 2, 4, 128, 90, 6, 64
    say(f"[graph] decode gate={gate}")
    x = prefill_inputs(B=N, T=T0 + steps, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=311 + gate)
    q, k, v = (torch.from_numpy(x[m]).to(DEV).to(torch.bfloat16) for m in ("q", "k", "v"))
    _, S_init = gla.liger_attn_prefill(q[:, :T0].contiguous(), k[:, :T0].contiguous(), v[:, :T0].contiguous(),
                                       gate, window, 0.5)
    ring = gla.KVRing.empty(N, H_kv, window, d, torch.bfloat16, DEV)
    gla.liger_kv_ring_fill(k[:, :T0].contiguous(), v[:, :T0].contiguous(), ring)
    torch.cuda.synchronize()
    init = dict(S=S_init.clone(), rk=ring.k.clone(), rv=ring.v.clone(), pos=ring.pos.clone(), sync=ring.sync.clone())
    qs = [q[:, T0 + i].contiguous() for i in range(steps)]
    ks = [k[:, T0 + i].contiguous() for i in range(steps)]
    vs = [v[:, T0 + i].contiguous() for i in range(steps)]
    S = S_init.clone()
    outs = [torch.empty_like(qs[0]) for _ in range(steps)]

    def reset():
        S.copy_(init["S"])
        ring.k.copy_(init["rk"])
        ring.v.copy_(init["rv"])
        ring.pos.copy_(init["pos"])
        ring.sync.copy_(init["sync"])
        for o in outs:
            o.fill_(float("nan"))

    def run():
        for i in range(steps):
            gla.liger_attn_decode_step(qs[i], ks[i], vs[i], S, ring, gate, 0.5, o=outs[i])

    reset()
    run()
    torch.cuda.synchronize()
    want = dict(o=[o.clone() for o in outs], S=S.clone(), rk=ring.k.clone(), rv=ring.v.clone(),
                pos=ring.pos.clone(), sync=ring.sync.clone())
    assert int(want["pos"][0].item()) == T0 + steps

    reset()
    graph = _capture(run)
    for r in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert torch.equal(outs[i], want["o"][i]), (r, i)
        assert torch.equal(S, want["S"]), r
        assert torch.equal(ring.k, want["rk"]) and torch.equal(ring.v, want["rv"]), r
        assert torch.equal(ring.pos, want["pos"]) and torch.equal(ring.sync, want["sync"]), r


@pytest.mark.parametrize("gate", [0, 1])
def test_prefill_replayed_from_a_graph(gate):
    B, T, H_kv, n_rep, d = 2, 700, 2, 4, 128
    say(f"[graph] prefill gate={gate}")
    x = prefill_inputs(B=B, T=T, H_q=H_kv * n_rep, H_kv=H_kv, d=d, dtype="bf16", seed=401 + gate)
    q, k, v = (torch.from_numpy(x[m]).to(DEV).to(torch.bfloat16) for m in ("q", "k", "v"))
    o = torch.empty_like(q)
    S_T = torch.empty(B, H_kv, d, d, dtype=torch.float32, device=DEV)
    ws = torch.empty(gla.liger_attn_prefill_workspace_size(B, T, H_kv * n_rep, H_kv, d, gla.LIGER_BF16),
                     dtype=torch.uint8, device=DEV)

    def run():
        gla.liger_attn_prefill(q, k, v, gate, 64, 0.5, o=o, S_T=S_T, workspace=ws)

    o.fill_(float("nan"))
    S_T.fill_(float("nan"))
    run()
    torch.cuda.synchronize()
    o_want, S_want = o.clone(), S_T.clone()
    assert not torch.isnan(o_want.float()).any() and not torch.isnan(S_want).any()
    graph = _capture(run)
    for r in range(REPLAYS):
        o.fill_(float("nan"))
        S_T.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_want), r
        assert torch.equal(S_T, S_want), r
