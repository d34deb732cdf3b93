"""Every named workload at full size, in the launch configuration the
benchmark times, against the CPU oracle: in full where the oracle runs in
seconds (single, dense, long_bf16, reduce), on sampled sequences / streams
otherwise (ragged, stream)."""
import gc

import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, TOL_BF16_OUT, announce, check, dev, host32, scan_header_error

pytestmark = pytest.mark.gpu
W = workloads.WORKLOADS


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


def test_ragged_sampled_sequences():
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
    rng = np.random.default_rng(123)
    pick = set(rng.choice(len(lengths), 40, replace=False).tolist())
    pick |= {0, 1, 2, len(lengths) - 1, int(lengths.argmax()), int(lengths.argmin())}
    qh = host32(q)
    worst = 0.0
    for s in sorted(pick):
        a, b = int(ho[s]), int(ho[s + 1])
        ref = oracle.scan_segmented(qh, host32(k[a:b]), host32(v[a:b]), np.array([0, b - a]), scale)
        worst = max(worst, check(o[a:b], ref, TOL[torch.float32], f"ragged sequence {s}"))
    # a contiguous run of sequences, crossing many tile boundaries
    a, b = int(ho[100]), int(ho[140])
    ref = oracle.scan_segmented(qh, host32(k[a:b]), host32(v[a:b]), ho[100:141] - a, scale)
    worst = max(worst, check(o[a:b], ref, TOL[torch.float32], "ragged sequences 100..139"))
    print(f"ragged: T={T} max scaled err over sampled sequences {worst:.3e}")


def test_stream_sampled_streams():
    w = W["stream"]
    sz = w.sizes
    S, H, d, T = sz["S"], sz["H"], sz["d"], sz["steps"]
    announce(f"workload stream: {w.describe()}")
    q, k, v = workloads.step_inputs(S, H, d, T, w.seed, device=dev())
    scale = workloads.default_scale(d)
    m, u, ww = aaren.new_state(S, H, d, device=dev())
    o = torch.empty(S, H, d, device=dev())
    sample = torch.from_numpy(np.sort(np.random.default_rng(5).choice(S, 512, replace=False))).to(dev())
    kept = []
    for t in range(T):
        aaren.aaren_step(q, k[t], v[t], m, u, ww, scale, o_t=o)
        kept.append(o[sample].clone())
    got = torch.stack(kept)                      # [T, 512, H, d]
    ks, vs = host32(k[:, sample]), host32(v[:, sample])
    del k, v
    st = oracle.state_init(len(sample), H, d)
    qh = host32(q)
    worst = 0.0
    for t in range(T):
        ref = oracle.step(qh, ks[t], vs[t], st, scale)
        worst = max(worst, check(got[t], ref, TOL[torch.float32], f"stream step {t}"))
    L = host32(m[sample]).astype(np.float64) + np.log(host32(u[sample]).astype(np.float64))
    Lr = st[0] + np.log(st[1])
    assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= 1e-5
    print(f"stream: max scaled err over 512 sampled streams x {T} steps {worst:.3e}")


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
    # dq sums B*N = 131072 terms per head: bound as in test_gpu_backward.dq_bound
    qh, kh = host32(q).astype(np.float64), host32(k).astype(np.float64)
    depth = 8 + 16 + -(-B * (N // 128) // 32) + 64
    for h in range(H):
        j = int(np.argmax(np.abs(qh[h])))
        sds = np.abs(rk[:, h, :, j]) / abs(qh[h, j])
        per_term = (depth * 2.0 ** -24 + 1e-5) * sds + 1e-5 / abs(qh[h, j])
        bound = (per_term[..., None] * np.abs(kh[:, h])).sum(axis=(0, 1))
        assert np.all(np.abs(host32(dq[h]) - rq[h]) <= bound)
    print(f"{name} gradients: dk {e_k:.3e} dv {e_v:.3e}")


def test_stream_appends_sampled_streams():
    """The stream workload's 256 tokens per stream as 16 appends of 16 (the
    append benchmark's launch shape), on 512 sampled streams."""
    w = W["stream"]
    sz = w.sizes
    S, H, d, T = sz["S"], sz["H"], sz["d"], sz["steps"]
    block = 16
    announce(f"workload stream, appends of {block}: {w.describe()}")
    q, k, v = workloads.step_inputs(S, H, d, T, w.seed, device=dev())
    scale = workloads.default_scale(d)
    m, u, ww = aaren.new_state(S, H, d, device=dev())
    o = torch.empty(block, S, H, d, device=dev())
    sample = torch.from_numpy(np.sort(np.random.default_rng(6).choice(S, 512, replace=False))).to(dev())
    kept = []
    for t0 in range(0, T, block):
        aaren.aaren_append(q, k[t0:t0 + block], v[t0:t0 + block], m, u, ww, scale, o=o)
        kept.append(o[:, sample].clone())
    got = torch.cat(kept)                        # [T, 512, H, d]
    ks, vs = host32(k[:, sample]), host32(v[:, sample])
    del k, v
    st = oracle.state_init(len(sample), H, d)
    ref = oracle.append(host32(q), ks, vs, st, scale)
    err = check(got, ref, TOL[torch.float32], "stream appends")
    L = host32(m[sample]).astype(np.float64) + np.log(host32(u[sample]).astype(np.float64))
    Lr = st[0] + np.log(st[1])
    assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= 1e-5
    print(f"stream appends: max scaled err over 512 sampled streams x {T} tokens {err:.3e}")


def test_self_attention_sampled_rows():
    """The causal self-attention workload at full size (the benchmark's call),
    rows at the start, the middle and the end of every (b,h) against the
    oracle's rows."""
    w = W["self_attn"]
    sz = w.sizes
    B, H, N, d = sz["B"], sz["H"], sz["N"], sz["d"]
    announce(f"workload self_attn: {w.describe()}")
    q, k, v = workloads.self_attention_inputs(B, H, N, d, w.seed, device=dev())
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_self_attention(q, k, v, scale, causal=bool(sz["causal"]), return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = host32(q), host32(k), host32(v)
    worst = 0.0
    for a, b in ((0, 128), (N // 2 - 64, N // 2 + 64), (N - 128, N)):
        ref, rl = oracle.self_attention(qh, kh, vh, scale, causal=bool(sz["causal"]), rows=(a, b),
                                        stats=True)
        worst = max(worst, check(o[:, :, a:b], ref, TOL[torch.bfloat16], f"rows {a}..{b}"))
        assert oracle.max_scaled_err(host32(lse[:, :, a:b]), rl) <= 1e-5
    print(f"self_attn: max scaled err over 384 rows x {B * H} heads {worst:.3e}")


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
    H=8, d=64) in full against the oracle, sequence by sequence; dq against
    the summation bound of test_gpu_backward.dq_bound."""
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
    depth = 8 + 16 + -(-(-(-T // 128)) // 32) + 64
    for h in range(H):
        j = int(np.argmax(np.abs(qh[h])))
        sds = np.abs(rk[:, h, j]) / abs(qh[h, j])
        per_term = (depth * 2.0 ** -24 + 1e-5) * sds + 1e-5 / abs(qh[h, j])
        bound = (per_term[:, None] * np.abs(kh[:, h].astype(np.float64))).sum(axis=0)
        assert np.all(np.abs(host32(dq[h]) - rq[h]) <= bound)
    print(f"packed gradients: T={T} dk {e_k:.3e} dv {e_v:.3e}")


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
