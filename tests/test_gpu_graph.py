"""The entry points under HIP graph capture.

The library allocates nothing and issues only kernel launches on the caller's
stream, so a whole step (prefill of a local and a global layer, the same with
log-sum-exp, the backward, decode against a ring and a linear cache, paged
decode) can be captured once and replayed.  Every replay must reproduce the
eager results bit for bit, with eager work and synchronisations between the
replays, and a replay after the inputs change in place must equal a fresh
eager call on the new inputs (the graph reads live memory).
"""
import sys

import numpy as np
import pytest
import torch

from attention_g2attn_prefill_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def g2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_g2attn_prefill_amd as mod
    return mod


def test_step_in_a_hip_graph_replays_bit_exact(g2):
    say("graph capture of a step")
    dev = torch.device("cuda:0")
    B, T, H, KVH, d, W = 1, 700, 4, 2, 256, 300
    kw = dict(query_scale=1 / 16, softcap=50.0, window=W)
    q = synth.draw((B, T, H, d), 61, 0, mul=3.0).to(dev)
    k = synth.draw((B, T, KVH, d), 61, 1, mul=3.0).to(dev)
    v = synth.draw((B, T, KVH, d), 61, 2).to(dev)
    dout = synth.draw((B, T, H, d), 61, 3).to(dev)
    # decode: 6 sequences, linear global cache of 1000 and a 300-slot ring
    DB, DS, RS = 6, 1000, W
    lens_np = np.array([1000, 999, 301, 300, 17, 1], np.int32)
    dq_ = synth.draw((DB, 1, H, d), 62, 0, mul=3.0).to(dev)
    lin_k = synth.draw((DB, DS, KVH, d), 62, 1)
    lin_v = synth.draw((DB, DS, KVH, d), 62, 2)
    ring_k = synth.ring_from_linear(lin_k, lens_np, RS, fill=0.0).to(dev)
    ring_v = synth.ring_from_linear(lin_v, lens_np, RS, fill=0.0).to(dev)
    kc, vc = lin_k.to(dev), lin_v.to(dev)
    lens = torch.from_numpy(lens_np).to(dev)
    pool_k, table = synth.paged_from_linear(lin_k, lens_np, 16, seed=63)
    pool_v, _ = synth.paged_from_linear(lin_v, lens_np, 16, seed=63)
    pool_k, pool_v, table = pool_k.to(dev), pool_v.to(dev), torch.from_numpy(table).to(dev)

    def buffers():
        return dict(
            loc=torch.empty_like(q), glo=torch.empty_like(q), lout=torch.empty_like(q),
            lse=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
            bws=torch.empty(g2.backward_workspace_bytes(B, T, T, H),
                            dtype=torch.uint8, device=dev),
            dring=torch.empty_like(dq_), dlin=torch.empty_like(dq_), dpag=torch.empty_like(dq_),
            ws1=torch.empty(g2.decode_workspace_bytes(DB, H, d, RS), dtype=torch.uint8, device=dev),
            ws2=torch.empty(g2.decode_workspace_bytes(DB, H, d, DS), dtype=torch.uint8, device=dev),
            ws3=torch.empty(g2.decode_paged_workspace_bytes(DB, H, d, table.shape[1], 16),
                            dtype=torch.uint8, device=dev))

    def step(o):
        g2.prefill(q, k, v, is_local=True, out=o["loc"], **kw)
        g2.prefill(q, k, v, is_local=False, out=o["glo"], **kw)
        g2.prefill_lse(q, k, v, is_local=True, out=o["lout"], lse=o["lse"], **kw)
        g2.prefill_backward(q, k, v, o["lout"], dout, o["lse"], is_local=True, dq=o["dq"],
                            dk=o["dk"], dv=o["dv"], workspace=o["bws"], **kw)
        g2.decode(dq_, ring_k, ring_v, lens, is_local=True, out=o["dring"], workspace=o["ws1"], **kw)
        g2.decode(dq_, kc, vc, lens, is_local=False, out=o["dlin"], workspace=o["ws2"], **kw)
        g2.decode_paged(dq_, pool_k, pool_v, table, lens, is_local=True, out=o["dpag"],
                        workspace=o["ws3"], **kw)

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    names = [n for n in eager if not n.startswith(("ws", "bws"))]
    for n in names:
        assert bool(torch.isfinite(eager[n].float()).all()), n

    graph_out = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(graph_out)  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(graph_out)
    torch.cuda.synchronize()

    for rep in range(3):
        for n in names:  # poison the graph's outputs so a replay that skips work shows
            graph_out[n].fill_(float("nan"))
        scratch = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(graph_out[n], eager[n]), f"replay {rep}: {n}"
        del scratch

    # change the inputs in place: the replay must follow them
    q.mul_(-1.0)
    dq_.mul_(0.5)
    fresh = buffers()
    step(fresh)
    graph.replay()
    torch.cuda.synchronize()
    for n in names:
        assert torch.equal(graph_out[n], fresh[n]), f"after input change: {n}"
        if n in ("loc", "glo", "dring"):
            assert not torch.equal(fresh[n], eager[n]), f"{n} did not change with its input"
    say("graph replays equal eager results")
