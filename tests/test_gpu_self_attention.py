"""Self-attention with one query per token on the GPU (aaren_self_attention,
bfloat16 inputs, matrix cores) against the CPU oracle's self-attention in
float64 on the same bfloat16 values."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
from _gpu import TOL, TOL_BF16_OUT, announce, check, dev, host32

pytestmark = pytest.mark.gpu


def inputs(B, H, N, d, seed, spread=1.0):
    g = torch.Generator(device=dev()).manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, device=dev())
    k = torch.randn(B, H, N, d, generator=g, device=dev()) * spread
    v = torch.randn(B, H, N, d, generator=g, device=dev())
    return tuple(t.to(torch.bfloat16).contiguous() for t in (q, k, v))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 64), (1, 2, 63, 64), (2, 2, 129, 64),
                                     (1, 1, 200, 128), (2, 3, 300, 128), (1, 2, 1000, 64),
                                     (1, 1, 1100, 128), (1, 1, 192, 128), (3, 3, 385, 128),
                                     (1, 1, 50, 128), (2, 1, 64, 128), (1, 2, 330, 128)])
def test_self_attention_matches_oracle(B, H, N, d, causal):
    announce(f"self-attention B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = inputs(B, H, N, d, seed=N + d)
    scale = float(np.float32(d ** -0.5))
    o, lse = aaren.aaren_self_attention(q, k, v, scale, causal=causal, return_lse=True)
    ref, rl = oracle.self_attention(host32(q), host32(k), host32(v), scale, causal=causal,
                                    stats=True)
    err = check(o, ref, TOL[torch.bfloat16], "o")
    err_l = oracle.max_scaled_err(host32(lse), rl)
    assert err_l <= 1e-5, err_l
    print(f"self-attention {B}x{H}x{N}x{d} causal={causal}: o {err:.2e} lse {err_l:.2e}")


def test_bf16_output_and_stretched_keys():
    """bf16 output (its own rounding bound) and keys stretched 8x (|s| ~ 40:
    the running maximum moves a lot between tiles)."""
    announce("self-attention bf16 out / spread")
    B, H, N, d = 1, 2, 700, 128
    q, k, v = inputs(B, H, N, d, seed=5, spread=8.0)
    scale = float(np.float32(d ** -0.5))
    ref = oracle.self_attention(host32(q), host32(k), host32(v), scale, causal=True)
    o32 = aaren.aaren_self_attention(q, k, v, scale)
    smax = float((q.float() @ k.float().transpose(-1, -2)).abs().max()) * scale
    tol = max(TOL[torch.bfloat16], 8 * smax * np.sqrt(d) * 2.0 ** -24)
    e32 = check(o32, ref, tol, "fp32 out")
    o16 = aaren.aaren_self_attention(q, k, v, scale, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    e16 = check(o16, ref, TOL_BF16_OUT, "bf16 out")
    print(f"spread |s| <= {smax:.0f}: fp32 out {e32:.2e}, bf16 out {e16:.2e}")


def test_equal_queries_reduce_to_the_scan():
    """Every query equal to q_h: causal self-attention is the many-to-many
    scan, and the GPU's two paths agree (both within tolerance of the
    oracle's scan)."""
    announce("self-attention equal queries")
    B, H, N, d = 2, 2, 777, 64
    _, k, v = inputs(B, H, N, d, seed=9)
    qh = torch.randn(H, d, device=dev()).to(torch.bfloat16)
    q = qh[None, :, None, :].expand(B, H, N, d).contiguous()
    o = aaren.aaren_self_attention(q, k, v)
    ref = oracle.scan(host32(qh), host32(k), host32(v), float(np.float32(d ** -0.5)))
    check(o, ref, TOL[torch.bfloat16], "equal queries vs oracle scan")
    o_scan = aaren.aaren_scan(qh, k, v)
    check(o, host32(o_scan).astype(np.float64), 2 * TOL[torch.bfloat16], "vs aaren_scan")


def test_empty_and_reproducible():
    announce("self-attention empty / determinism")
    z = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev())
    out = aaren.aaren_self_attention(z, z, z)
    assert out.shape == (1, 2, 0, 64)
    q, k, v = inputs(1, 2, 513, 64, seed=11)
    a = aaren.aaren_self_attention(q, k, v)
    for _ in range(3):
        assert torch.equal(a, aaren.aaren_self_attention(q, k, v))


@pytest.mark.parametrize("d", [64, 128])
def test_value_magnitudes(d):
    """Values far outside fp16's range, per head: 2^40, 2^-40, bf16
    subnormals (2^-130), unit scale, and unit scale with one element at 2^20.
    The value product runs in fp16 after a power-of-two scale per (b,h);
    attention is linear in V, so o / s is held to the unit-scale bound."""
    announce(f"self-attention value magnitudes d={d}")
    B, H, N = 1, 5, 333
    q, k, _ = inputs(B, H, N, d, seed=13)
    g = torch.Generator(device=dev()).manual_seed(14)
    s = torch.tensor([2.0 ** 40, 2.0 ** -40, 2.0 ** -130, 1.0, 1.0], dtype=torch.float64)
    v32 = torch.randn(B, H, N, d, generator=g, device=dev())
    v32 = v32 * s.to(torch.float32).to(dev())[None, :, None, None]
    v32[0, 4, 100, 7] = 2.0 ** 20
    v = v32.to(torch.bfloat16).contiguous()
    assert 0 < float(v[0, 2].float().abs().max()) < 2.0 ** -126  # subnormal head
    scale = float(np.float32(d ** -0.5))
    for causal in (True, False):
        o = host32(aaren.aaren_self_attention(q, k, v, scale, causal=causal)).astype(np.float64)
        ref = oracle.self_attention(host32(q), host32(k), host32(v), scale, causal=causal)
        sn = s.numpy()[None, :, None, None]
        err = oracle.max_scaled_err(o / sn, ref / sn)
        assert err <= TOL[torch.bfloat16], (causal, err)
        print(f"value magnitudes d={d} causal={causal}: o/s {err:.2e}")


def test_longest_sequence():
    """N = 2^22, the longest the entry point takes, at d = 128: the tile
    copies' buffer byte counts reach 2^30 there. Sampled rows at the start,
    the middle and the end (the last rows read every key of the head)."""
    B, H, N, d = 1, 1, 1 << 22, 128
    announce(f"self-attention longest sequence B={B} H={H} N={N} d={d} causal")
    q, k, v = inputs(B, H, N, d, seed=23)
    scale = float(np.float32(d ** -0.5))
    o, lse = aaren.aaren_self_attention(q, k, v, scale, return_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = host32(q), host32(k), host32(v)
    worst = 0.0
    for a, b in ((0, 8), (N // 2 - 4, N // 2 + 4), (N - 8, N)):
        ref, rl = oracle.self_attention(qh, kh, vh, scale, causal=True, rows=(a, b), stats=True)
        worst = max(worst, check(o[:, :, a:b], ref, TOL[torch.bfloat16], f"rows {a}..{b}"))
        assert oracle.max_scaled_err(host32(lse[:, :, a:b]), rl) <= 1e-5
    print(f"self-attention N=2^22: max scaled err over 24 rows {worst:.3e}")
