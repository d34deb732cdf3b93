"""The calls that launch plain kernels (no look-back epoch, no memset) under
HIP graph capture: self-attention, the reduction and the step, each captured
once and replayed several times with the program's own eager work and
synchronisations between replays; every replay must equal the eager result
bit for bit."""
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import workloads
from _gpu import announce, dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _noise():
    """Eager work between replays: it must not disturb what the graph reads."""
    x = torch.randn(1 << 20, device=dev())
    torch.cuda.synchronize()
    return float(x.sum())


def test_self_attention_in_a_graph():
    announce("graph: self-attention")
    B, H, N, d = 1, 2, 1000, 128
    g = torch.Generator(device=dev()).manual_seed(21)
    q, k, v = (torch.randn(B, H, N, d, generator=g, device=dev()).to(torch.bfloat16)
               for _ in range(3))
    ws = torch.empty(aaren.aaren_self_attention_workspace_size(B, H, N, d), dtype=torch.uint8,
                     device=dev())
    ref = aaren.aaren_self_attention(q, k, v, workspace=ws).clone()
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_self_attention(q, k, v, out=out, workspace=ws)
    for _ in range(REPLAYS):
        out.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(aaren.aaren_self_attention(q, k, v, workspace=ws), ref)


def test_reduce_in_a_graph():
    announce("graph: reduce")
    B, H, N, d = 2, 3, 50000, 128
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=22, device=dev())
    ws = torch.empty(aaren.aaren_reduce_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    ref = aaren.aaren_reduce(q, k, v, workspace=ws).clone()
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_reduce(q, k, v, out=out, workspace=ws)
    for _ in range(REPLAYS):
        out.fill_(7.0)
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(aaren.aaren_reduce(q, k, v, workspace=ws), ref)


def test_steps_in_a_graph():
    """One captured step replayed T times is T steps: the state and the last
    output equal T eager steps."""
    announce("graph: step")
    S, H, d, T = 1000, 4, 64, 5
    q, k, v = workloads.step_inputs(S, H, d, T, seed=23, device=dev())
    kt, vt = torch.empty_like(k[0]), torch.empty_like(v[0])
    m, u, w = aaren.new_state(S, H, d, device=dev())
    for t in range(T):
        o_ref = aaren.aaren_step(q, k[t], v[t], m, u, w)
    ref = (m.clone(), u.clone(), w.clone(), o_ref.clone())
    m2, u2, w2 = aaren.new_state(S, H, d, device=dev())
    o = torch.empty_like(o_ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_step(q, kt, vt, m2, u2, w2, o_t=o)
    aaren.aaren_state_init(m2, u2, w2)  # capture does not run the step
    for t in range(T):
        kt.copy_(k[t])
        vt.copy_(v[t])
        _noise()
        graph.replay()
        torch.cuda.synchronize()
    assert torch.equal(m2, ref[0]) and torch.equal(u2, ref[1]) and torch.equal(w2, ref[2])
    assert torch.equal(o, ref[3])
