"""The strided scan (token-major tensors) and one or two stacked Aaren layers
(rocBLAS projection + scan) on the GPU against the CPU oracle."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, TOL_BF16_OUT, announce, check, dev, host32, scan_header_error

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,N,d", [(2, 3, 300, 64), (1, 2, 1000, 128), (3, 1, 1, 64)])
def test_scan_on_token_major_tensors(B, H, N, d, dt):
    """k, v stored [B,N,H,d] (as a projection writes them), viewed as
    [B,H,N,d]; output in the same layout."""
    announce(f"strided scan B={B} H={H} N={N} d={d} {dt}")
    torch_dt = torch.float32 if dt == "f32" else torch.bfloat16
    g = torch.Generator(device=dev()).manual_seed(N + d)
    k = torch.randn(B, N, H, d, generator=g, device=dev()).to(torch_dt)
    v = torch.randn(B, N, H, d, generator=g, device=dev()).to(torch_dt)
    q = torch.randn(H, d, generator=g, device=dev()).to(torch_dt)
    kv, vv = k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)
    o, lse = aaren.aaren_scan_strided(q, kv, vv, return_lse=True)
    assert o.stride() == kv.stride()
    ref, _, rl = oracle.scan(host32(q), host32(kv.contiguous()), host32(vv.contiguous()),
                             workloads.default_scale(d), stats=True)
    check(o, ref, TOL[torch_dt], "strided scan")
    assert oracle.max_scaled_err(host32(lse), rl) <= 1e-5


def _layer_inputs(B, N, Dm, H, d, seed):
    g = torch.Generator(device=dev()).manual_seed(seed)
    x = torch.randn(B, N, Dm, generator=g, device=dev()).to(torch.bfloat16)
    w = (torch.randn(Dm, 2 * H * d, generator=g, device=dev()) / Dm ** 0.5).to(torch.bfloat16)
    q = torch.randn(H, d, generator=g, device=dev())
    return x, w, q


@pytest.mark.parametrize("B,N,Dm,H,d", [(2, 300, 96, 3, 64), (1, 700, 256, 2, 128),
                                        (2, 1, 64, 1, 64)])
def test_layer_matches_oracle(B, N, Dm, H, d):
    """fp32 output: the GEMM's fp32 accumulation moves K and V by about
    Dm 2^-24 relative, far inside 1e-5; bf16 output: its rounding bound."""
    announce(f"layer B={B} N={N} Dm={Dm} H={H} d={d}")
    x, w, q = _layer_inputs(B, N, Dm, H, d, seed=N + Dm)
    scale = workloads.default_scale(d)
    ws = torch.zeros(aaren.aaren_layer_workspace_size(B, N, Dm, H, d), dtype=torch.uint8, device=dev())
    o32 = aaren.aaren_layer_forward(x, w, q, scale, out_dtype=torch.float32, workspace=ws)
    o16 = aaren.aaren_layer_forward(x, w, q, scale, workspace=ws)
    torch.cuda.synchronize()
    assert scan_header_error(ws) == 0
    assert o16.dtype == torch.bfloat16 and o16.shape == (B, N, H, d)
    ref = oracle.layer_forward(host32(x), host32(w), host32(q), scale, out_bf16=False)
    e32 = check(o32, ref, TOL[torch.float32], "layer fp32 out")
    # against the unrounded value: the GPU's one rounding is at most half an ulp
    e16 = check(o16, ref, TOL_BF16_OUT, "layer bf16 out")
    print(f"layer {B}x{N}x{Dm} H={H} d={d}: fp32 {e32:.2e} bf16 {e16:.2e}")


@pytest.mark.parametrize("spread", [60.0])
def test_layer_with_stretched_scores(spread):
    """q scaled so that the largest |score| is `spread`: the scores reach the
    scan as x (W_K q), with W_K q carried into the product as three bf16
    parts. With all three the scores are off by the fp32 rounding of two dot
    products (length Dm in the product, d in W_K q), so the bound scales with
    the spread: 8 |s| (sqrt(Dm) + sqrt(d)) 2^-24. W_K q rounded to bf16 once
    would move the scores by about |s| 2^-9 (0.1 here), far past it; two
    parts (about |s| 2^-17) would stay inside this bound."""
    announce(f"layer stretched scores {spread}")
    B, N, Dm, H, d = 1, 800, 256, 2, 64
    x, w, q = _layer_inputs(B, N, Dm, H, d, seed=77)
    scale = workloads.default_scale(d)
    xh, wh, qh = (host32(t).astype(np.float64) for t in (x, w, q))
    kh = (xh @ wh[:, :H * d]).reshape(B, N, H, d)
    s = scale * np.einsum("bnhd,hd->bnh", kh, qh)
    q = q * float(spread / np.abs(s).max())
    o32 = aaren.aaren_layer_forward(x, w, q, scale, out_dtype=torch.float32)
    ref = oracle.layer_forward(host32(x), host32(w), host32(q), scale, out_bf16=False)
    bound = max(1e-5, 8 * spread * (Dm ** 0.5 + d ** 0.5) * 2.0 ** -24)
    err = check(o32, ref, bound, "layer stretched scores")
    print(f"layer stretched scores {spread}: fp32 {err:.2e} (bound {bound:.1e})")


def test_two_stacked_layers():
    """The second layer takes the first one's bf16 output (rounded on both
    sides: that rounding is part of the stack's definition). Where the GPU's
    and the oracle's first-layer outputs fall on different sides of a bf16
    rounding boundary (about 1 element in 4000) the second layer's keys and
    values move by 2^-8 |x_j w_jk|, which moves its outputs by far less than
    their own rounding. The last layer is compared unrounded: bound, its
    rounding 2^-8 plus 1e-4 per layer."""
    announce("two stacked layers")
    B, N, H, d = 2, 500, 2, 64
    x, w1, q1 = _layer_inputs(B, N, H * d, H, d, seed=1)
    _, w2, q2 = _layer_inputs(B, N, H * d, H, d, seed=2)
    scale = workloads.default_scale(d)
    h1 = aaren.aaren_layer_forward(x, w1, q1, scale)
    h2 = aaren.aaren_layer_forward(h1.reshape(B, N, H * d), w2, q2, scale)
    r1 = oracle.layer_forward(host32(x), host32(w1), host32(q1), scale)
    r2 = oracle.layer_forward(r1.reshape(B, N, H * d), host32(w2), host32(q2), scale,
                              out_bf16=False)
    err = check(h2, r2, TOL_BF16_OUT + 2e-4, "two layers")
    print(f"two stacked layers: max scaled err {err:.2e}")


def test_layer_empty_is_a_noop():
    announce("layer empty")
    x = torch.zeros(0, 5, 64, dtype=torch.bfloat16, device=dev())
    w = torch.zeros(64, 128, dtype=torch.bfloat16, device=dev())
    q = torch.zeros(1, 64, device=dev())
    assert aaren.aaren_layer_forward(x, w, q).shape == (0, 5, 1, 64)
