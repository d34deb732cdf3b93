"""Every named workload at full size, in the launch configuration the
benchmark times, against the CPU oracle, every output element: large
outputs in chunks (sequences, steps, row blocks), the oracle's float64
reference compared on the device (gpu_scaled_err)."""
import gc

import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import (TOL, TOL_BF16_OUT, announce, check, dev, dq_tol, gpu_scaled_err, host32,
                  progress, scan_header_error)

pytestmark = pytest.mark.gpu
W = workloads.WORKLOADS


def _dq_report(got, ref) -> str:
    """Where dq's scaled error peaks: that error, the absolute error and the
    reference there, and the largest |dq|."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    sc = err / (1 + np.abs(ref))
    i = np.unravel_index(int(sc.argmax()), sc.shape)
    return (f"dq worst scaled {sc[i]:.2e} (|err| {err[i]:.2e} at |dq| {abs(ref[i]):.2e}; "
            f"max |dq| {np.abs(ref).max():.2e})")


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["single", "dense"])
def test_dense_workloads_in_full(name):
    w = W[name]
    sz = w.sizes
    announce(f"workload {name}: {w.describe()}")
    q, k, v = workloads.dense_inputs(sz["B"], sz["H"], sz["N"], sz["d"], w.seed, device=dev())
    scale = workloads.default_scale(sz["d"])
    o = aaren.aaren_scan(q, k, v, scale)
    ref = oracle.scan(host32(q), host32(k), host32(v), scale)
    err = check(o, ref, TOL[torch.float32], name)
    print(f"{name}: max scaled err {err:.3e}")


def test_long_bf16_in_full():
    w = W["long_bf16"]
    sz = w.sizes
    announce(f"workload long_bf16: {w.describe()}")
    q, k, v = workloads.dense_inputs(sz["B"], sz["H"], sz["N"], sz["d"], w.seed, device=dev(),
                                     dtype="bf16", score_span=w.score_span)
    scale = workloads.default_scale(sz["d"])
    ws = torch.zeros(aaren.aaren_scan_workspace_size(*k.shape), dtype=torch.uint8, device=dev())
    o = aaren.aaren_scan(q, k, v, scale, workspace=ws)
    torch.cuda.synchronize()
    assert scan_header_error(ws) == 0
    qh = host32(q)
    worst = 0.0
    for b in range(sz["B"]):  # one batch row at a time keeps host memory small
        ref = oracle.scan(qh, host32(k[b:b + 1]), host32(v[b:b + 1]), scale)
        worst = max(worst, check(o[b:b + 1], ref, TOL[torch.bfloat16], f"long_bf16 b={b}"))
    print(f"long_bf16: max scaled err {worst:.3e}")


def test_ragged_in_full():
    """All 4096 sequences of the packed workload, in chunks of consecutive
    sequences of about 2^18 tokens (each chunk's reference is the oracle's
    packed scan of those sequences)."""
    w = W["ragged"]
    sz = w.sizes
    announce(f"workload ragged: {w.describe()}")
    lengths = workloads.segment_lengths(sz["num_seqs"], sz["max_len"], w.seed)
    q, k, v, offs = workloads.segmented_inputs(lengths, sz["H"], sz["d"], w.seed, device=dev())
    scale = workloads.default_scale(sz["d"])
    T = int(lengths.sum())
    ws = torch.zeros(aaren.aaren_scan_segmented_workspace_size(len(lengths), T, sz["H"], sz["d"]),
                     dtype=torch.uint8, device=dev())
    o = aaren.aaren_scan_segmented(q, k, v, offs, scale, workspace=ws)
    torch.cuda.synchronize()
    assert scan_header_error(ws) == 0
    ho = offs.cpu().numpy()
    qh = host32(q)
    # chunk boundaries: the first sequence start at or after every 2^18 tokens
    cuts = np.unique(np.concatenate([np.searchsorted(ho, np.arange(0, T, 1 << 18)),
                                     [len(lengths)]]))
    worst = 0.0
    for c, (s0, s1) in enumerate(zip(cuts[:-1], cuts[1:])):
        a, b = int(ho[s0]), int(ho[s1])
        ref = oracle.scan_segmented(qh, host32(k[a:b]), host32(v[a:b]), ho[s0:s1 + 1] - a, scale)
        err = gpu_scaled_err(o[a:b], ref)
        assert err <= TOL[torch.float32], f"sequences {s0}..{s1 - 1}: {err:.3e}"
        worst = max(worst, err)
        if c % 16 == 15:
            progress(f"ragged: sequences 0..{s1 - 1} of {len(lengths)} checked")
    print(f"ragged: T={T}, all {len(lengths)} sequences, max scaled err {worst:.3e}")


def test_stream_in_full():
    """All 262,144 x 4 streams for all 256 steps: the oracle steps every
    stream in lockstep (float64 state), each step's o_t compared in full."""
    w = W["stream"]
    sz = w.sizes
    S, H, d, T = sz["S"], sz["H"], sz["d"], sz["steps"]
    announce(f"workload stream: {w.describe()}")
    q, k, v = workloads.step_inputs(S, H, d, T, w.seed, device=dev())
    scale = workloads.default_scale(d)
    m, u, ww = aaren.new_state(S, H, d, device=dev())
    o = torch.empty(S, H, d, device=dev())
    st = oracle.state_init(S, H, d)
    qh = host32(q)
    worst = 0.0
    for t in range(T):
        aaren.aaren_step(q, k[t], v[t], m, u, ww, scale, o_t=o)
        ref = oracle.step(qh, host32(k[t]), host32(v[t]), st, scale)
        err = gpu_scaled_err(o, ref)
        assert err <= TOL[torch.float32], f"step {t}: {err:.3e}"
        worst = max(worst, err)
        if t % 32 == 31:
            progress(f"stream: steps 0..{t} checked")
    L = host32(m).astype(np.float64) + np.log(host32(u).astype(np.float64))
    Lr = st[0] + np.log(st[1])
    assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= 1e-5
    mr = st[0]                                   # m: the running maximum of the scores
    assert np.max(np.abs(host32(m) - mr) / (1 + np.abs(mr))) <= 1e-5
    print(f"stream: all {S} streams x {H} heads x {T} steps, max scaled err {worst:.3e}")


def test_reduce_in_full():
    w = W["reduce"]
    sz = w.sizes
    announce(f"workload reduce: {w.describe()}")
    q, k, v = workloads.reduce_inputs(sz["B"], sz["H"], sz["N"], sz["d"], w.seed, device=dev())
    scale = workloads.default_scale(sz["d"])
    o, m, u = aaren.aaren_reduce(q, k, v, scale, stats=True)
    ref, rm, rl = oracle.reduce(host32(q), host32(k), host32(v), scale, stats=True)
    err = check(o, ref, TOL[torch.float32], "reduce")
    L = host32(m).astype(np.float64) + np.log(host32(u).astype(np.float64))
    assert np.max(np.abs(L - rl) / (1 + np.abs(rl))) <= 1e-5
    print(f"reduce: max scaled err {err:.3e}")


@pytest.mark.parametrize("name", ["dense", "backward_bf16"])
def test_dense_gradients_in_full(name):
    """Gradients at the dense batch's full size (the backward benches' shape),
    float32 and with bf16 q, K, V and output gradients."""
    w = W[name]
    sz = w.sizes
    B, H, N, d = sz["B"], sz["H"], sz["N"], sz["d"]
    announce(f"workload {name} gradients: {w.describe()}")
    q, k, v = workloads.dense_inputs(B, H, N, d, w.seed, device=dev(), dtype=w.dtype)
    g = torch.randn(B, H, N, d, device=dev(), generator=torch.Generator(device=dev()).manual_seed(w.seed + 100))
    g = g.to(k.dtype)
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan(q, k, v, scale, return_lse=True)
    dq, dk, dv = aaren.aaren_scan_backward(q, k, v, o, g, lse, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.scan_backward(host32(q), host32(k), host32(v), host32(g), scale)
    e_k = check(dk, rk, 1e-5, "dk")
    e_v = check(dv, rv, 1e-5, "dv")
    got_q = host32(dq).astype(np.float64)
    e_q = oracle.max_scaled_err(got_q, rq)
    tol_q = dq_tol(B * N)
    assert e_q <= tol_q, f"dq: {e_q:.3e}"
    # The check would see one lane group's 8-row partial lost: remove rows
    # 8..15 of batch row 3's first tile from head h's sum (the terms
    # scale ds_i k_i, with scale ds_i = dk_ij / q_j along q's largest j).
    qh, kh = host32(q).astype(np.float64), host32(k).astype(np.float64)
    for h in range(H):
        j = int(np.argmax(np.abs(qh[h])))
        lost = (rk[3, h, 8:16, j] / qh[h, j])[:, None] * kh[3, h, 8:16]
        planted = got_q.copy()
        planted[h] -= lost.sum(axis=0)
        assert oracle.max_scaled_err(planted, rq) > tol_q, h
    print(f"{name} gradients: dq {e_q:.3e} dk {e_k:.3e} dv {e_v:.3e}; {_dq_report(got_q, rq)}")


def test_stream_appends_in_full():
    """The stream workload's 256 tokens per stream as 16 appends of 16 (the
    append benchmark's launch shape), every stream and token against the
    oracle's steps."""
    w = W["stream"]
    sz = w.sizes
    S, H, d, T = sz["S"], sz["H"], sz["d"], sz["steps"]
    block = 16
    announce(f"workload stream, appends of {block}: {w.describe()}")
    q, k, v = workloads.step_inputs(S, H, d, T, w.seed, device=dev())
    scale = workloads.default_scale(d)
    m, u, ww = aaren.new_state(S, H, d, device=dev())
    o = torch.empty(block, S, H, d, device=dev())
    st = oracle.state_init(S, H, d)
    qh = host32(q)
    worst = 0.0
    for t0 in range(0, T, block):
        aaren.aaren_append(q, k[t0:t0 + block], v[t0:t0 + block], m, u, ww, scale, o=o)
        for i in range(block):
            ref = oracle.step(qh, host32(k[t0 + i]), host32(v[t0 + i]), st, scale)
            err = gpu_scaled_err(o[i], ref)
            assert err <= TOL[torch.float32], f"token {t0 + i}: {err:.3e}"
            worst = max(worst, err)
        if t0 % 64 == 48:
            progress(f"stream appends: tokens 0..{t0 + block - 1} checked")
    L = host32(m).astype(np.float64) + np.log(host32(u).astype(np.float64))
    Lr = st[0] + np.log(st[1])
    assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= 1e-5
    print(f"stream appends: all {S} streams x {H} heads x {T} tokens, max scaled err {worst:.3e}")


def test_self_attention_in_full():
    """The causal self-attention workload at full size (the benchmark's
    call): every row of every (b,h) and its log-normaliser against the
    oracle, in blocks of 2048 query rows."""
    w = W["self_attn"]
    sz = w.sizes
    B, H, N, d = sz["B"], sz["H"], sz["N"], sz["d"]
    announce(f"workload self_attn: {w.describe()}")
    q, k, v = workloads.self_attention_inputs(B, H, N, d, w.seed, device=dev())
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_self_attention(q, k, v, scale, causal=bool(sz["causal"]), return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = host32(q), host32(k), host32(v)
    worst = worst_l = 0.0
    for a in range(0, N, 2048):
        b = min(N, a + 2048)
        ref, rl = oracle.self_attention(qh, kh, vh, scale, causal=bool(sz["causal"]), rows=(a, b),
                                        stats=True)
        err = gpu_scaled_err(o[:, :, a:b], ref)
        err_l = gpu_scaled_err(lse[:, :, a:b], rl)
        assert err <= TOL[torch.bfloat16], f"rows {a}..{b - 1}: {err:.3e}"
        assert err_l <= 1e-5, f"lse rows {a}..{b - 1}: {err_l:.3e}"
        worst, worst_l = max(worst, err), max(worst_l, err_l)
        progress(f"self_attn: rows 0..{b - 1} of {N} checked")
    print(f"self_attn: all {N} rows x {B * H} heads, max scaled err {worst:.3e}, "
          f"lse {worst_l:.3e}")


def test_layer_stack_in_full():
    """The benchmark's four stacked layers at full size against the oracle's
    stack (each layer's bf16 output feeds the next on both sides; the last
    layer's GPU output, rounded once, against the unrounded oracle: bound as
    for two layers, 2^-8 plus 1e-4 per layer)."""
    w = W["layer"]
    sz = w.sizes
    B, N, Dm, H, d, L = sz["B"], sz["N"], sz["Dm"], sz["H"], sz["d"], sz["layers"]
    announce(f"workload layer: {w.describe()}")
    x, ws_, qs = workloads.layer_inputs(B, N, Dm, H, d, L, w.seed, device=dev())
    scale = workloads.default_scale(d)
    h = x
    for layer in range(L):
        h = aaren.aaren_layer_forward(h.reshape(B, N, -1), ws_[layer], qs[layer], scale)
    torch.cuda.synchronize()
    r = host32(x)
    for layer in range(L):  # bf16 between layers, the last one unrounded
        r = oracle.layer_forward(r.reshape(B, N, -1), host32(ws_[layer]), host32(qs[layer]), scale,
                                 out_bf16=layer < L - 1)
    err = check(h, r, TOL_BF16_OUT + L * 1e-4, "layer stack")
    print(f"layer stack: max scaled err {err:.3e}")


def test_packed_gradients_in_full():
    """Gradients of the packed workload (1024 sequences, lengths U{1..8192},
    H=8, d=64) in full against the oracle, sequence by sequence; dq to
    dq_tol(T)."""
    w = W["ragged_backward"]
    sz = w.sizes
    H, d = sz["H"], sz["d"]
    announce(f"workload ragged_backward: {w.describe()}")
    lengths = workloads.segment_lengths(sz["num_seqs"], sz["max_len"], w.seed)
    q, k, v, offs = workloads.segmented_inputs(lengths, H, d, w.seed, device=dev())
    T = int(lengths.sum())
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan_segmented(q, k, v, offs, scale, return_lse=True)
    g = torch.randn(T, H, d, device=dev(),
                    generator=torch.Generator(device=dev()).manual_seed(w.seed + 100))
    dq, dk, dv = aaren.aaren_scan_segmented_backward(q, k, v, o, g, lse, offs, scale)
    torch.cuda.synchronize()
    del o, lse
    qh, kh, vh, gh = host32(q), host32(k), host32(v), host32(g)
    del v, g
    rq, rk, rv = oracle.scan_segmented_backward(qh, kh, vh, gh, offs.cpu().numpy(), scale)
    e_k = check(dk, rk, 1e-5, "packed dk")
    del dk
    e_v = check(dv, rv, 1e-5, "packed dv")
    del dv, rv
    e_q = oracle.max_scaled_err(host32(dq), rq)
    print(f"packed gradients: T={T} dq {e_q:.3e} dk {e_k:.3e} dv {e_v:.3e}; "
          f"{_dq_report(host32(dq), rq)}")
    assert e_q <= dq_tol(T), f"dq: {e_q:.3e}"


def test_mean_query_in_full():
    """The mean-query workload at full size (B=4, H=8, N=65536, d=128), in the
    benchmark's call: every (b,h) against the oracle."""
    w = W["mean_query"]
    sz = w.sizes
    B, H, N, d = sz["B"], sz["H"], sz["N"], sz["d"]
    announce(f"workload mean_query: {w.describe()}")
    hq, k, v = workloads.mean_query_inputs(B, H, N, d, w.seed, device=dev())
    scale = workloads.default_scale(d)
    ws = torch.empty(aaren.aaren_mean_query_attention_workspace_size(B, H, N, d),
                     dtype=torch.uint8, device=dev())
    o = aaren.aaren_mean_query_attention(hq, k, v, scale, workspace=ws)
    ref = oracle.mean_query_attention(host32(hq), host32(k), host32(v), scale)
    err = check(o, ref, TOL[torch.float32], "mean_query")
    print(f"mean_query: max scaled err {err:.3e}")
