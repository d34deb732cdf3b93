"""Long look-back chains under repetition: the backward over one stream of
2^20 rows (8192 tiles, carried from the end), and a packed batch whose one
long sequence spans thousands of tiles among thousands of short ones. 100
calls on one workspace must be bitwise identical (the carries are left folds
in a fixed order whatever the timing) and agree with the oracle."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, announce, check, dev, host32, scan_header_error

pytestmark = pytest.mark.gpu

REPEATS = 100


def test_backward_one_stream_of_8192_tiles():
    announce("backward 8192-tile chain x100")
    B, H, N, d = 1, 1, 1 << 20, 64
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=15, device=dev())
    g = torch.randn(B, H, N, d, device=dev(), generator=torch.Generator(device=dev()).manual_seed(16))
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan(q, k, v, scale, return_lse=True)
    ws = torch.zeros(aaren.aaren_scan_backward_workspace_size(B, H, N, d), dtype=torch.uint8,
                     device=dev())
    first = [t.clone() for t in aaren.aaren_scan_backward(q, k, v, o, g, lse, scale, workspace=ws)]
    dq, dk, dv = (torch.empty_like(t) for t in first)
    for _ in range(REPEATS - 1):
        aaren.aaren_scan_backward(q, k, v, o, g, lse, scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(dq, first[0]) and torch.equal(dk, first[1]) and torch.equal(dv, first[2])
    assert scan_header_error(ws) == 0
    rq, rk, rv = oracle.scan_backward(host32(q), host32(k), host32(v), host32(g), scale)
    check(first[1], rk, 1e-5, "dk, 8192-tile chain")
    check(first[2], rv, 1e-5, "dv, 8192-tile chain")


def test_packed_long_and_short_sequences():
    announce("packed long + short sequences x100")
    rng = np.random.default_rng(17)
    lengths = np.concatenate([rng.integers(1, 40, size=3000), [1 << 20],
                              rng.integers(1, 40, size=3000)]).astype(np.int64)
    H, d = 2, 64
    q, k, v, offs = workloads.segmented_inputs(lengths, H, d, seed=18, device=dev())
    T = int(lengths.sum())
    ws = torch.zeros(aaren.aaren_scan_segmented_workspace_size(len(lengths), T, H, d),
                     dtype=torch.uint8, device=dev())
    first = aaren.aaren_scan_segmented(q, k, v, offs, workspace=ws).clone()
    o = torch.empty_like(first)
    for _ in range(REPEATS - 1):
        aaren.aaren_scan_segmented(q, k, v, offs, out=o, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, first)
    assert scan_header_error(ws) == 0
    # the oracle on the long sequence and on 200 sampled short ones
    ho = offs.cpu().numpy()
    scale = workloads.default_scale(d)
    picks = sorted(set(rng.integers(0, len(lengths), size=200).tolist()) | {3000})
    for s in picks:
        a, b = int(ho[s]), int(ho[s + 1])
        sub = [np.ascontiguousarray(host32(x[a:b]).transpose(1, 0, 2)[None]) for x in (k, v)]
        ref = oracle.scan(host32(q), sub[0], sub[1], scale)[0].transpose(1, 0, 2)
        check(first[a:b], ref, TOL[torch.float32], f"sequence {s} of length {b - a}")


def test_perturbed_schedules_give_the_same_bits(monkeypatch):
    """With AAREN_STRESS=1 every tile pauses a pseudo-random time after taking
    its ticket and after publishing its aggregate, so tiles publish and walk
    in unusual orders; the forward, backward and packed results must still be
    bitwise those of unperturbed calls."""
    announce("look-back under perturbed schedules")
    B, H, N, d = 1, 2, 1 << 19, 64
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=19, device=dev())
    g = torch.randn(B, H, N, d, device=dev(), generator=torch.Generator(device=dev()).manual_seed(20))
    o, lse = aaren.aaren_scan(q, k, v, return_lse=True)
    grads = aaren.aaren_scan_backward(q, k, v, o, g, lse)
    lengths = np.array([3, 70000, 1, 129, 5000, 2, 100000, 17], np.int64)
    qp, kp, vp, offs = workloads.segmented_inputs(lengths, H, d, seed=21, device=dev())
    op = aaren.aaren_scan_segmented(qp, kp, vp, offs)
    torch.cuda.synchronize()
    monkeypatch.setenv("AAREN_STRESS", "1")
    for _ in range(3):
        o2, lse2 = aaren.aaren_scan(q, k, v, return_lse=True)
        grads2 = aaren.aaren_scan_backward(q, k, v, o, g, lse)
        op2 = aaren.aaren_scan_segmented(qp, kp, vp, offs)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(lse2, lse)
        assert all(torch.equal(a, b) for a, b in zip(grads2, grads))
        assert torch.equal(op2, op)
    monkeypatch.delenv("AAREN_STRESS")


def test_graph_replays_under_perturbed_schedules(monkeypatch):
    """A dense scan captured into a graph with AAREN_STRESS=1 (tiles pause at
    random; the calls take device-side epochs) and replayed ten times: every
    replay equals the unperturbed eager result bit for bit."""
    announce("graph replays under perturbed schedules")
    B, H, N, d = 2, 4, 1 << 17, 64
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=34, device=dev())
    ref = aaren.aaren_scan(q, k, v)
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    out = torch.empty_like(ref)
    aaren.aaren_scan(q, k, v, out=out, workspace=ws)
    torch.cuda.synchronize()
    monkeypatch.setenv("AAREN_STRESS", "1")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        aaren.aaren_scan(q, k, v, out=out, workspace=ws)
    monkeypatch.delenv("AAREN_STRESS")
    for _ in range(10):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert scan_header_error(ws) == 0
