"""Calls from several host threads at once, each thread on a stream of its
own (default priority) with the binding's per-stream workspaces: the dense
and packed scans, the gradients, the reduction, steps, self-attention and
the layer, repeated, must give exactly the results of the same calls made
from one thread. ctypes releases the interpreter lock during library calls,
so the library's host code (validation, epochs, workspace bookkeeping, the
layer's rocBLAS handle) runs concurrently."""
import threading

import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import workloads
from _gpu import announce, dev

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 3


def _case(seed):
    g = torch.Generator(device=dev()).manual_seed(seed)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device=dev())
    B, H, N, d = 2, 2, 1500, 64
    c = {"q": rnd(H, d), "k": rnd(B, H, N, d), "v": rnd(B, H, N, d), "g": rnd(B, H, N, d)}
    lengths = [300, 0, 1200, 7]
    c["offsets"] = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64, device=dev())
    T = sum(lengths)
    c["kp"], c["vp"] = rnd(T, H, d), rnd(T, H, d)
    c["kt"], c["vt"] = rnd(6, 500, H, d), rnd(6, 500, H, d)
    c["sq"], c["sk"], c["sv"] = (rnd(1, 2, 700, 128).to(torch.bfloat16) for _ in range(3))
    x, w, q = workloads.layer_inputs(2, 600, 128, 2, 64, 1, seed, device=dev())
    c["x"], c["w"], c["lq"] = x, w[0], q[0]
    return c


def _run(c):
    out = {}
    out["o"], out["lse"] = aaren.aaren_scan(c["q"], c["k"], c["v"], return_lse=True)
    out["dq"], out["dk"], out["dv"] = aaren.aaren_scan_backward(c["q"], c["k"], c["v"], out["o"],
                                                                c["g"], out["lse"])
    out["op"] = aaren.aaren_scan_segmented(c["q"], c["kp"], c["vp"], c["offsets"])
    out["r"] = aaren.aaren_reduce(c["q"], c["k"], c["v"])
    m, u, w = aaren.new_state(500, 2, 64, device=dev())
    for t in range(c["kt"].shape[0]):
        out["step"] = aaren.aaren_step(c["q"], c["kt"][t], c["vt"][t], m, u, w)
    out["w"] = w
    out["sa"] = aaren.aaren_self_attention(c["sq"], c["sk"], c["sv"])
    out["layer"] = aaren.aaren_layer_forward(c["x"], c["w"], c["lq"])
    return out


def test_concurrent_threads_match_one_thread():
    announce(f"threads: {THREADS} host threads x {ROUNDS} rounds, one stream each")
    cases = [_case(50 + i) for i in range(THREADS)]
    refs = [_run(c) for c in cases]          # one thread, the current stream
    torch.cuda.synchronize()
    results = [[None] * ROUNDS for _ in range(THREADS)]
    errors = []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev())
            with torch.cuda.stream(s):
                start.wait()
                for r in range(ROUNDS):
                    results[i][r] = _run(cases[i])
            s.synchronize()
        except Exception as e:  # reported below with the thread's index
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(THREADS):
        for r in range(ROUNDS):
            for key, ref in refs[i].items():
                assert torch.equal(results[i][r][key], ref), f"thread {i} round {r}: {key}"
