"""Multi-token append on the GPU (aaren_append) against the CPU oracle's
append (T successive single-pair updates in float64)."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, TOL_BF16_OUT, announce, check, dev, host32

pytestmark = pytest.mark.gpu


def _lse(m, u):
    return host32(m).astype(np.float64) + np.log(host32(u).astype(np.float64))


def _tol(in_dt, out_dt):
    return TOL_BF16_OUT if out_dt == torch.bfloat16 else TOL[in_dt]


@pytest.mark.parametrize("S,H,T,d,in_dt,out_dt", [
    (5, 3, 1, 64, torch.float32, torch.float32),
    (7, 2, 13, 64, torch.float32, torch.float32),
    (3, 4, 40, 128, torch.float32, torch.float32),
    (1000, 4, 17, 64, torch.float32, torch.float32),
    (300, 2, 9, 128, torch.bfloat16, torch.float32),
    (64, 3, 20, 64, torch.bfloat16, torch.bfloat16),
    (33, 1, 8, 64, torch.float32, torch.bfloat16),
])
def test_append_matches_oracle(S, H, T, d, in_dt, out_dt):
    """A first block from the empty state, then a second block on top of it."""
    announce(f"append S={S} H={H} T={T} d={d} {in_dt} -> {out_dt}")
    T0 = 5
    dt = "bf16" if in_dt == torch.bfloat16 else "f32"
    q, k, v = workloads.step_inputs(S, H, d, T0 + T, seed=40 + T, device=dev(), dtype=dt)
    scale = workloads.default_scale(d)
    m, u, w = aaren.new_state(S, H, d, device=dev())
    o0 = aaren.aaren_append(q, k[:T0], v[:T0], m, u, w, scale, out_dtype=out_dt)
    o1 = aaren.aaren_append(q, k[T0:], v[T0:], m, u, w, scale, out_dtype=out_dt)
    st = oracle.state_init(S, H, d)
    qh, kh, vh = host32(q), host32(k), host32(v)
    r0 = oracle.append(qh, kh[:T0], vh[:T0], st, scale)
    r1 = oracle.append(qh, kh[T0:], vh[T0:], st, scale)
    tol = _tol(in_dt, out_dt)
    check(o0, r0, tol, "first block")
    err = check(o1, r1, tol, "second block")
    L = _lse(m, u)
    Lr = st[0] + np.log(st[1])
    assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= TOL[in_dt]
    print(f"append {S}x{H}x{T}x{d}: max scaled err {err:.2e}")


def test_append_equals_steps():
    """One append of T tokens == T aaren_step calls, bit for bit: both absorb
    each pair with the same fp32 arithmetic."""
    announce("append vs steps")
    for (S, H, T, d, dt) in [(129, 4, 21, 64, "f32"), (40, 2, 9, 128, "bf16")]:
        q, k, v = workloads.step_inputs(S, H, d, T, seed=50, device=dev(), dtype=dt)
        m1, u1, w1 = aaren.new_state(S, H, d, device=dev())
        m2, u2, w2 = aaren.new_state(S, H, d, device=dev())
        steps = torch.stack([aaren.aaren_step(q, k[t], v[t], m1, u1, w1) for t in range(T)])
        o = aaren.aaren_append(q, k, v, m2, u2, w2)
        torch.cuda.synchronize()
        assert torch.equal(steps, o)
        assert torch.equal(m1, m2) and torch.equal(u1, u2) and torch.equal(w1, w2)


def test_append_block_sizes_agree():
    """40 tokens in one call, as 8 + 32, and as 1 + 39 + 0: the same scan."""
    announce("append block sizes")
    S, H, T, d = 77, 2, 40, 128
    q, k, v = workloads.step_inputs(S, H, d, T, seed=51, device=dev())
    st = oracle.state_init(S, H, d)
    ref = oracle.append(host32(q), host32(k), host32(v), st, workloads.default_scale(d))
    for cuts in ([40], [8, 32], [1, 39, 0]):
        m, u, w = aaren.new_state(S, H, d, device=dev())
        outs, t0 = [], 0
        for n in cuts:
            outs.append(aaren.aaren_append(q, k[t0:t0 + n], v[t0:t0 + n], m, u, w))
            t0 += n
        check(torch.cat(outs), ref, 1e-5, f"blocks {cuts}")
        L = _lse(m, u)
        Lr = st[0] + np.log(st[1])
        assert np.max(np.abs(L - Lr) / (1 + np.abs(Lr))) <= 1e-5


def test_append_empty_and_without_output():
    """T = 0 changes nothing; emit=False leaves o alone and updates the state
    exactly as emit=True does."""
    announce("append empty / no output")
    S, H, T, d = 40, 3, 12, 64
    q, k, v = workloads.step_inputs(S, H, d, T, seed=52, device=dev())
    m, u, w = aaren.new_state(S, H, d, device=dev())
    aaren.aaren_append(q, k[:4], v[:4], m, u, w)
    before = (m.clone(), u.clone(), w.clone())
    out = torch.full((0, S, H, d), 3.0, device=dev())
    aaren.aaren_append(q, k[:0], v[:0], m, u, w, o=out)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((m, u, w), before))
    m2, u2, w2 = (t.clone() for t in before)
    o = aaren.aaren_append(q, k[4:], v[4:], m, u, w)
    assert aaren.aaren_append(q, k[4:], v[4:], m2, u2, w2, emit=False) is None
    torch.cuda.synchronize()
    assert torch.equal(m, m2) and torch.equal(u, u2) and torch.equal(w, w2)
    assert o.shape == (T - 4, S, H, d)


def test_append_large_score_spread():
    """Keys stretched 40x (|s| up to ~200): the state's maximum moves by
    hundreds between blocks; bound 8 |s|max sqrt(d) 2^-24 as for the scan."""
    announce("append spread")
    S, H, T, d = 200, 2, 30, 64
    q, k, v = workloads.step_inputs(S, H, d, T, seed=53, device=dev())
    k = k * 40.0
    scale = workloads.default_scale(d)
    m, u, w = aaren.new_state(S, H, d, device=dev())
    o = torch.cat([aaren.aaren_append(q, k[:13], v[:13], m, u, w, scale),
                   aaren.aaren_append(q, k[13:], v[13:], m, u, w, scale)])
    st = oracle.state_init(S, H, d)
    ref = oracle.append(host32(q), host32(k), host32(v), st, scale)
    smax = float(np.abs(np.einsum("tshd,hd->tsh", host32(k), host32(q))).max()) * scale
    tol = max(1e-5, 8 * smax * 8 * 2.0 ** -24)
    err = check(o, ref, tol, "spread")
    print(f"append spread: |s| <= {smax:.0f}, tol {tol:.1e}, err {err:.2e}")
