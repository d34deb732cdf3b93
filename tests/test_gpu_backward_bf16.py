"""Gradients with bfloat16 q, K, V and output gradients (dense and packed):
against the CPU oracle's float64 gradients of the same bfloat16 values, and
bit for bit against the float32 backward of those values widened (bf16 ->
fp32 is exact and the arithmetic after it is the same)."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import announce, dev, dq_tol, host32
from test_gpu_backward import errs

pytestmark = pytest.mark.gpu

bf16 = torch.bfloat16


def _dense(B, H, N, d, seed):
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=seed, device=dev(), dtype="bf16")
    g = torch.randn(B, H, N, d, device=dev(),
                    generator=torch.Generator(device=dev()).manual_seed(seed + 1)).to(bf16)
    return q, k, v, g


@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 64), (2, 3, 127, 64), (2, 1, 129, 64),
                                     (1, 2, 1000, 64), (1, 1, 300, 128), (2, 2, 1000, 128)])
def test_bf16_backward_matches_oracle(B, H, N, d):
    announce(f"bf16 backward B={B} H={H} N={N} d={d}")
    q, k, v, g = _dense(B, H, N, d, seed=170 + N)
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan(q, k, v, scale, return_lse=True)
    assert o.dtype == torch.float32
    got = aaren.aaren_scan_backward(q, k, v, o, g, lse, scale)
    torch.cuda.synchronize()
    ref = oracle.scan_backward(host32(q), host32(k), host32(v), host32(g), scale)
    e_dq, e_dk, e_dv = errs(got, ref)
    print(f"bf16 backward {B}x{H}x{N}x{d}: dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    # inputs widen exactly, so the float32 bounds apply
    assert e_dk <= 1e-5 and e_dv <= 1e-5, (e_dk, e_dv)
    assert e_dq <= dq_tol(B * N), e_dq


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_backward_is_the_widened_float32_backward(d):
    announce(f"bf16 backward == widened fp32 backward d={d}")
    B, H, N = 2, 3, 1500
    q, k, v, g = _dense(B, H, N, d, seed=200 + d)
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan(q, k, v, scale, return_lse=True)
    a = aaren.aaren_scan_backward(q, k, v, o, g, lse, scale)
    b = aaren.aaren_scan_backward(q.float(), k.float(), v.float(), o, g.float(), lse, scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("lengths,H,d", [
    ([3, 1, 400, 0, 77, 129, 128, 1000], 3, 64),
    ([700, 0, 0, 333, 1, 1, 2048], 2, 128),
])
def test_bf16_packed_backward(lengths, H, d):
    announce(f"bf16 packed backward lengths={lengths[:8]} H={H} d={d}")
    seed = 300 + len(lengths) + d
    q, k, v, offs = workloads.segmented_inputs(np.array(lengths, np.int64), H, d, seed,
                                               device=dev())
    q, k, v = q.to(bf16), k.to(bf16), v.to(bf16)
    g = torch.randn(k.shape, device=dev(),
                    generator=torch.Generator(device=dev()).manual_seed(seed)).to(bf16)
    scale = workloads.default_scale(d)
    o, lse = aaren.aaren_scan_segmented(q, k, v, offs, scale, return_lse=True)
    dq, dk, dv = aaren.aaren_scan_segmented_backward(q, k, v, o, g, lse, offs, scale)
    w = aaren.aaren_scan_segmented_backward(q.float(), k.float(), v.float(), o, g.float(), lse,
                                            offs, scale)
    torch.cuda.synchronize()
    assert torch.equal(dq, w[0]) and torch.equal(dk, w[1]) and torch.equal(dv, w[2])
    rq, rk, rv = oracle.scan_segmented_backward(host32(q), host32(k), host32(v), host32(g),
                                                offs.cpu().numpy(), scale)
    e_dq, e_dk, e_dv = errs((dq, dk, dv), (rq, rk, rv))
    print(f"bf16 packed backward H={H} d={d}: dq {e_dq:.2e} dk {e_dk:.2e} dv {e_dv:.2e}")
    assert e_dk <= 1e-5 and e_dv <= 1e-5, (e_dk, e_dv)
    assert e_dq <= dq_tol(sum(lengths)), e_dq


def test_bf16_backward_rejects_mixed_dtypes():
    q, k, v, g = _dense(1, 1, 10, 64, seed=1)
    o, lse = aaren.aaren_scan(q, k, v, return_lse=True)
    with pytest.raises(TypeError):
        aaren.aaren_scan_backward(q, k, v, o.to(bf16), g, lse)   # o must be float32
    with pytest.raises(TypeError):
        aaren.aaren_scan_backward(q, k, v, o, g.float(), lse)    # dout with k's dtype
