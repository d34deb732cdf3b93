"""Calls under HIP graph capture, each captured once and replayed several
times with the program's own eager work and synchronisations between
replays; every replay must equal the eager result bit for bit.

Self-attention, the reduction and the step launch plain kernels. The scans
and their gradients exchange states between tiles tagged with an epoch:
captured, they advance an epoch word in the workspace on the device before
each launch, so replays on new inputs (copied into the captured tensors) are
checked against eager calls on those inputs, made on the same workspace in
between (eager calls use host epochs, which never meet the graph's)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import workloads
from _gpu import announce, dev, scan_header_error

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

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


def _refill(gen, *ts):
    """New values in captured input tensors (same storage)."""
    for t in ts:
        t.copy_(torch.randn(t.shape, generator=gen, device=dev()).to(t.dtype))


def test_dense_scan_in_a_graph():
    announce("graph: dense scan")
    B, H, N, d = 2, 3, 3000, 64            # several tiles per stream
    g = torch.Generator(device=dev()).manual_seed(31)
    q, k, v = (torch.empty(*shape, device=dev()) for shape in ((H, d), (B, H, N, d), (B, H, N, d)))
    _refill(g, q, k, v)
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    o, lse = torch.empty(B, H, N, d, device=dev()), torch.empty(B, H, N, device=dev())
    aaren.aaren_scan(q, k, v, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan(q, k, v, out=o, lse=lse, workspace=ws)
    for _ in range(REPLAYS):
        _refill(g, q, k, v)
        o.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        ref, ref_l = aaren.aaren_scan(q, k, v, workspace=ws, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_l)
        assert scan_header_error(ws) == 0


@pytest.mark.parametrize("half", ["0", "1"])
def test_dense_scan_of_two_rounds_in_a_graph(half, monkeypatch):
    """A call of two rounds of resident workgroups (32 x 8 streams of 1000
    rows: 1024 full tiles, or 1536 with each stream ending in half tiles),
    captured with either tiling; replays equal eager calls made with the
    same tiling."""
    monkeypatch.setenv("AAREN_HALF_TILES", half)
    announce(f"graph: dense scan 32x8x1000, half tiles {half}")
    B, H, N, d = 32, 8, 1000, 64
    g = torch.Generator(device=dev()).manual_seed(37)
    q, k, v = (torch.empty(*shape, device=dev()) for shape in ((H, d), (B, H, N, d), (B, H, N, d)))
    _refill(g, q, k, v)
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    o = torch.empty(B, H, N, d, device=dev())
    aaren.aaren_scan(q, k, v, out=o, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan(q, k, v, out=o, workspace=ws)
    for _ in range(REPLAYS):
        _refill(g, q, k, v)
        o.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        ref = aaren.aaren_scan(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)
        assert scan_header_error(ws) == 0


def test_graph_replays_between_calls_of_other_shapes():
    """A scan of 256 streams captured into a graph, with eager scans of 8
    streams on the same workspace before every replay: the small calls' tile
    states cover the bytes the large call counts tickets in, so each replay
    must clear its own counters (the capture records that), and the eager
    calls after a replay must clear theirs. Every replay and every eager call
    equals the result on a workspace of its own, and the error word stays
    clear."""
    announce("graph: 256-stream scan replayed between 8-stream eager scans")
    d, N = 64, 1024
    g = torch.Generator(device=dev()).manual_seed(34)
    qb, kb, vb = (torch.randn(*s_, generator=g, device=dev())
                  for s_ in ((8, d), (32, 8, N, d), (32, 8, N, d)))
    qs, ks, vs = (torch.randn(*s_, generator=g, device=dev())
                  for s_ in ((8, d), (1, 8, N, d), (1, 8, N, d)))
    ref_b = aaren.aaren_scan(qb, kb, vb, workspace=torch.zeros(
        aaren.aaren_scan_workspace_size(32, 8, N, d), dtype=torch.uint8, device=dev())).clone()
    ref_s = aaren.aaren_scan(qs, ks, vs, workspace=torch.zeros(
        aaren.aaren_scan_workspace_size(1, 8, N, d), dtype=torch.uint8, device=dev())).clone()
    ws = torch.zeros(aaren.aaren_scan_workspace_size(32, 8, N, d), dtype=torch.uint8,
                     device=dev())
    ob = torch.empty_like(kb)
    aaren.aaren_scan(qb, kb, vb, out=ob, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan(qb, kb, vb, out=ob, workspace=ws)
    for _ in range(REPLAYS):
        assert torch.equal(aaren.aaren_scan(qs, ks, vs, workspace=ws), ref_s)
        ob.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, ref_b)
        assert aaren.aaren_workspace_status(ws) == 0
        assert torch.equal(aaren.aaren_scan(qs, ks, vs, workspace=ws), ref_s)
        assert torch.equal(aaren.aaren_scan(qb, kb, vb, workspace=ws), ref_b)
        assert aaren.aaren_workspace_status(ws) == 0


def test_packed_scan_in_a_graph():
    announce("graph: packed scan")
    H, d = 2, 128
    lengths = [1, 700, 0, 2500, 33]
    offsets = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64, device=dev())
    T = sum(lengths)
    g = torch.Generator(device=dev()).manual_seed(32)
    q = torch.empty(H, d, device=dev())
    k, v = (torch.empty(T, H, d, device=dev(), dtype=torch.bfloat16) for _ in range(2))
    _refill(g, q, k, v)
    q = q.to(torch.bfloat16)
    ws = torch.zeros(aaren.aaren_scan_segmented_workspace_size(len(lengths), T, H, d),
                     dtype=torch.uint8, device=dev())
    o = torch.empty(T, H, d, device=dev())
    aaren.aaren_scan_segmented(q, k, v, offsets, out=o, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan_segmented(q, k, v, offsets, out=o, workspace=ws)
    for _ in range(REPLAYS):
        _refill(g, k, v)
        o.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        ref = aaren.aaren_scan_segmented(q, k, v, offsets, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)
        assert scan_header_error(ws) == 0


def test_scan_gradients_in_a_graph():
    announce("graph: dense scan gradients")
    B, H, N, d = 2, 2, 2000, 64
    g = torch.Generator(device=dev()).manual_seed(33)
    q, k, v, dout = (torch.empty(*shape, device=dev())
                     for shape in ((H, d), (B, H, N, d), (B, H, N, d), (B, H, N, d)))
    _refill(g, q, k, v, dout)
    o, lse = aaren.aaren_scan(q, k, v, return_lse=True)
    wsb = torch.zeros(aaren.aaren_scan_backward_workspace_size(B, H, N, d), dtype=torch.uint8,
                      device=dev())
    dq, dk, dv = torch.empty(H, d, device=dev()), torch.empty_like(k), torch.empty_like(v)
    aaren.aaren_scan_backward(q, k, v, o, dout, lse, dq=dq, dk=dk, dv=dv, workspace=wsb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan_backward(q, k, v, o, dout, lse, dq=dq, dk=dk, dv=dv, workspace=wsb)
    for _ in range(REPLAYS):
        _refill(g, q, k, v, dout)
        o2, lse2 = aaren.aaren_scan(q, k, v, return_lse=True)   # the forward of the new inputs
        o.copy_(o2)
        lse.copy_(lse2)
        dk.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        rq, rk, rv = aaren.aaren_scan_backward(q, k, v, o, dout, lse, workspace=wsb)
        torch.cuda.synchronize()
        assert torch.equal(dq, rq) and torch.equal(dk, rk) and torch.equal(dv, rv)
        assert scan_header_error(wsb) == 0


def test_layer_in_a_graph():
    """The layer (rocBLAS product, then the strided scan) captured after one
    eager call on the device, replayed on new x."""
    announce("graph: layer")
    B, N, Dm, H, d = 2, 1500, 256, 4, 64
    x, w, q = workloads.layer_inputs(B, N, Dm, H, d, 1, 41, device=dev())
    w, q = w[0], q[0]
    wsp = torch.zeros(aaren.aaren_layer_workspace_size(B, N, Dm, H, d), dtype=torch.uint8, device=dev())
    o = torch.empty(B, N, H, d, dtype=torch.bfloat16, device=dev())
    aaren.aaren_layer_forward(x, w, q, out=o, workspace=wsp)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_layer_forward(x, w, q, out=o, workspace=wsp)
    g = torch.Generator(device=dev()).manual_seed(42)
    for _ in range(REPLAYS):
        _refill(g, x)
        o.zero_()
        _noise()
        graph.replay()
        torch.cuda.synchronize()
        ref = aaren.aaren_layer_forward(x, w, q, workspace=wsp)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)


_INIT_THEN_CAPTURE = """
import ctypes, torch, exact_softmax_attention_02_amd as aaren, workloads
dev = torch.device("cuda:0")
x, w, q = workloads.layer_inputs(1, 300, 128, 2, 64, 1, 43, device=dev)
w, q = w[0], q[0]
wsp = torch.zeros(aaren.aaren_layer_workspace_size(1, 300, 128, 2, 64), dtype=torch.uint8, device=dev)
o = torch.full((1, 300, 2, 64), 7.0, dtype=torch.bfloat16, device=dev)
P = lambda t: ctypes.c_void_p(t.data_ptr())
st = aaren.lib.aaren_layer_forward(P(x), P(w), P(q), P(o), 1, 300, 128, 2, 64, 0.125,
                                   aaren.AAREN_BF16, P(wsp), wsp.numel(), None)
torch.cuda.synchronize()
assert st == aaren.AAREN_ERR_UNSUPPORTED, st
assert "aaren_init" in aaren.aaren_last_error()
assert bool((o == 7.0).all())
print("refused before aaren_init")
aaren.aaren_init()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    aaren.aaren_layer_forward(x, w, q, out=o, workspace=wsp)
print("first layer call captured")
for _ in range(3):
    o.zero_()
    graph.replay()
    torch.cuda.synchronize()
    ref = aaren.aaren_layer_forward(x, w, q, workspace=wsp)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
print("replays equal eager calls")
"""


def test_layer_needs_init_and_is_captured_after_it():
    """In a fresh process a layer call before aaren_init is refused with
    UNSUPPORTED and touches nothing; after aaren_init (which creates the
    rocBLAS handle) the very first layer call can be captured, and its
    replays equal eager calls. A child process, so that no earlier call of
    the test session has initialised the device."""
    announce("graph: layer refused before aaren_init, captured after it (child process)")
    env = dict(os.environ, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", _INIT_THEN_CAPTURE], capture_output=True,
                       text=True, env=env, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    for line in ("refused before aaren_init", "first layer call captured",
                 "replays equal eager calls"):
        assert line in r.stdout, r.stdout
