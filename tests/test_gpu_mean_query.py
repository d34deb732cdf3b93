"""Mean-query (global-aggregation) attention on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, announce, check, dev, host32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,N,d", [(1, 1, 1, 64), (2, 3, 1000, 64), (1, 2, 5000, 128),
                                     (3, 1, 70000, 64)])
def test_mean_query_matches_oracle(B, H, N, d, dt):
    announce(f"mean query B={B} H={H} N={N} d={d} {dt}")
    torch_dt = torch.float32 if dt == "f32" else torch.bfloat16
    g = torch.Generator(device=dev()).manual_seed(N + d)
    hq, k, v = (torch.randn(B, H, N, d, generator=g, device=dev()).to(torch_dt) for _ in range(3))
    hq = hq + 0.5  # a mean query of some size, so the weights are not all equal
    scale = workloads.default_scale(d)
    o, gq = aaren.aaren_mean_query_attention(hq, k, v, scale, return_query=True)
    ref, rg = oracle.mean_query_attention(host32(hq), host32(k), host32(v), scale, stats=True)
    # the GPU's g is the float64 mean rounded once to float32: within half an ulp
    assert np.allclose(host32(gq), rg, rtol=2.0 ** -23, atol=0)
    err = check(o, ref, TOL[torch_dt], "mean query")
    print(f"mean query {B}x{H}x{N}x{d} {dt}: {err:.2e}")


def test_mean_query_reproducible():
    announce("mean query determinism")
    hq, k, v = (torch.randn(2, 2, 30000, 64, device=dev()) for _ in range(3))
    a = aaren.aaren_mean_query_attention(hq, k, v)
    for _ in range(3):
        assert torch.equal(a, aaren.aaren_mean_query_attention(hq, k, v))
