"""Dense many-to-many scan on the GPU against the CPU oracle.

Sizes span several tiles (256 rows for d=64 fp32 and d=128 bf16, 128 for
d=128 fp32, 512 for d=64 bf16) with ragged tails."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
import workloads
from _gpu import TOL, TOL_BF16_OUT, announce, check, dev, host32, scan_header_error

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("d,ind,outd", [(64, "f32", "f32"), (128, "bf16", "f32"),
                                        (128, "f32", "f32"), (64, "bf16", "f32"),
                                        (64, "f32", "bf16"), (128, "bf16", "bf16")])
@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 1, 2), (2, 3, 17), (1, 2, 255), (1, 1, 256),
                                   (2, 1, 257), (1, 3, 1000), (3, 2, 2049)])
def test_scan_small(B, H, N, d, ind, outd):
    announce(f"scan B={B} H={H} N={N} d={d} in={ind} out={outd}")
    scale = workloads.default_scale(d)
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=100 + N, device=dev(), dtype=ind)
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    o = aaren.aaren_scan(q, k, v, scale, out_dtype=DT[outd], workspace=ws)
    ref = oracle.scan(host32(q), host32(k), host32(v), scale)
    tol = TOL_BF16_OUT if outd == "bf16" else TOL[DT[ind]]
    check(o, ref, tol, "scan")
    assert scan_header_error(ws) == 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [383, 384, 385, 511, 512, 513, 640, 700, 767, 768, 769, 1100])
def test_scan_stream_ends_in_half_tiles(d, N, monkeypatch):
    """fp32 streams ending in half tiles (the last full tile split in two, the
    rows after it in halves; forced here, the library takes them for calls of
    several rounds of resident workgroups): lengths around the full and half
    tile edges (256 and 128 rows at d=64, 128 and 64 at d=128), values and
    the log-normaliser against the oracle."""
    monkeypatch.setenv("AAREN_HALF_TILES", "1")
    announce(f"scan half tiles N={N} d={d}")
    B, H = 2, 3
    scale = workloads.default_scale(d)
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=300 + N, device=dev())
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    o, lse = aaren.aaren_scan(q, k, v, scale, workspace=ws, return_lse=True)
    ref, _, ref_lse = oracle.scan(host32(q), host32(k), host32(v), scale, stats=True)
    check(o, ref, TOL[torch.float32], "scan")
    check(lse, ref_lse, TOL[torch.float32], "lse")
    assert scan_header_error(ws) == 0


@pytest.mark.parametrize("mode", ["0", "1"])
def test_scan_many_rounds_with_and_without_half_tiles(mode, monkeypatch):
    """A call of two rounds of resident workgroups (32 x 8 streams of 1000
    rows: 1024 tiles, 1536 with halves), both tilings against the oracle."""
    monkeypatch.setenv("AAREN_HALF_TILES", mode)
    announce(f"scan 32x8x1000 half tiles {mode}")
    B, H, N, d = 32, 8, 1000, 64
    scale = workloads.default_scale(d)
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=41, device=dev())
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    o = aaren.aaren_scan(q, k, v, scale, workspace=ws)
    check(o, oracle.scan(host32(q), host32(k), host32(v), scale), TOL[torch.float32], "scan")
    assert scan_header_error(ws) == 0


@pytest.mark.parametrize("d,ind", [(64, "f32"), (128, "bf16"), (128, "f32")])
@pytest.mark.parametrize("half", ["0", "1"])
def test_scan_bf16_output_is_the_rounded_fp32_output(d, ind, half, monkeypatch):
    """The bf16 output is the fp32 output of the same call rounded to nearest
    even (torch's conversion), bit for bit: the kernels round on the chip."""
    monkeypatch.setenv("AAREN_HALF_TILES", half)
    announce(f"scan bf16 output rounding d={d} in={ind} half={half}")
    B, H, N = 2, 3, 1500
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=55, device=dev(), dtype=ind)
    o32 = aaren.aaren_scan(q, k, v, out_dtype=torch.float32)
    o16 = aaren.aaren_scan(q, k, v, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_scan_single_token_is_exact():
    announce("scan single token exact")
    q, k, v = workloads.dense_inputs(4, 8, 1, 64, seed=7, device=dev())
    o = aaren.aaren_scan(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, v)


def test_scan_equal_scores_running_mean():
    announce("scan q=0 running mean")
    _, k, v = workloads.dense_inputs(2, 2, 777, 64, seed=8, device=dev())
    q = torch.zeros(2, 64, device=dev())
    o = aaren.aaren_scan(q, k, v)
    vv = host32(v).astype(np.float64)
    ref = np.cumsum(vv, axis=2) / np.arange(1, 778)[None, None, :, None]
    check(o, ref, 1e-5, "running mean")


@pytest.mark.parametrize("spread", [80.0, 1000.0])
def test_scan_large_score_spread(spread):
    """Scores far beyond exp's range: only a running maximum keeps this finite
    (and a tile-wide maximum would underflow early rows). The fp32 dot product
    itself is off by about |s| sqrt(d) 2^-24, which moves every weight by that
    factor, so the bound scales with the spread: 8 |s| sqrt(d) 2^-24."""
    announce(f"scan spread {spread}")
    B, H, N, d = 1, 2, 1500, 64
    g = torch.Generator(device=dev()).manual_seed(9)
    q = torch.randn(H, d, generator=g, device=dev())
    k = torch.randn(B, H, N, d, generator=g, device=dev())
    v = torch.randn(B, H, N, d, generator=g, device=dev())
    s = (k @ q[None, :, :, None]).squeeze(-1) * 0.125
    k = k * (spread / s.abs().amax(-1, keepdim=True))[..., None]
    o = aaren.aaren_scan(q, k, v, 0.125)
    ref = oracle.scan(host32(q), host32(k), host32(v), 0.125)
    check(o, ref, max(1e-5, 8 * spread * d ** 0.5 * 2.0 ** -24), f"spread {spread}")


def test_scan_ascending_scores_every_row_a_new_maximum():
    """Each row raises the running maximum (rescale on every row). Scores reach
    |s| = 300, so fp32 score rounding (about |s| 2^-24 per score, one nonzero
    coordinate per dot product) bounds the error: 8 |s| 2^-24."""
    announce("scan ascending scores")
    N, d = 600, 64
    q = torch.zeros(1, d, device=dev())
    q[0, 0] = 1.0
    k = torch.zeros(1, 1, N, d, device=dev())
    k[0, 0, :, 0] = torch.linspace(-300, 300, N, device=dev())
    v = torch.randn(1, 1, N, d, device=dev(), generator=torch.Generator(device=dev()).manual_seed(3))
    o = aaren.aaren_scan(q, k, v, 1.0)
    ref = oracle.scan(host32(q), host32(k), host32(v), 1.0)
    check(o, ref, max(1e-5, 8 * 300 * 2.0 ** -24), "ascending")


def test_scan_repeat_is_bitwise_deterministic_and_workspace_reusable():
    """Thousands of tiles chained by look-back; repeated calls on one workspace
    (epochs advance) give bitwise-identical results."""
    announce("scan repeat determinism")
    B, H, N, d = 2, 2, 65536, 64
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=11, device=dev())
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    first = aaren.aaren_scan(q, k, v, workspace=ws)
    for _ in range(20):
        again = aaren.aaren_scan(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(first, again)
    assert scan_header_error(ws) == 0
    counters = ws[256:256 + B * H * 128].view(torch.int32)
    assert int(counters.abs().sum().item()) == 0  # every ticket counter wrapped back to 0
    ref = oracle.scan(host32(q), host32(k), host32(v), workloads.default_scale(d))
    check(first, ref, 1e-5, "long chain")


def test_scan_workspace_shared_by_shapes():
    """One workspace serves calls of different shapes in turn."""
    announce("scan workspace across shapes")
    ws = torch.zeros(aaren.aaren_scan_workspace_size(4, 4, 3000, 128), dtype=torch.uint8,
                     device=dev())
    for (B, H, N, d) in [(4, 4, 3000, 128), (1, 1, 5, 64), (2, 3, 999, 64), (4, 4, 3000, 128)]:
        q, k, v = workloads.dense_inputs(B, H, N, d, seed=N, device=dev())
        o = aaren.aaren_scan(q, k, v, workspace=ws)
        ref = oracle.scan(host32(q), host32(k), host32(v), workloads.default_scale(d))
        check(o, ref, 1e-5, f"shape {(B, H, N, d)}")
    assert scan_header_error(ws) == 0


def test_scan_on_a_side_stream():
    announce("scan side stream")
    q, k, v = workloads.dense_inputs(2, 2, 1000, 64, seed=12, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = aaren.aaren_scan(q, k, v)
    s.synchronize()
    ref = oracle.scan(host32(q), host32(k), host32(v), workloads.default_scale(64))
    check(o, ref, 1e-5, "side stream")


def test_scan_convex_hull_large():
    """Property at a size the oracle is not run on: each output coordinate lies
    within the running min/max of the values."""
    announce("scan convex hull")
    q, k, v = workloads.dense_inputs(4, 4, 8192, 64, seed=13, device=dev())
    o = aaren.aaren_scan(q, k, v)
    lo = torch.cummin(v, dim=2).values
    hi = torch.cummax(v, dim=2).values
    torch.cuda.synchronize()
    assert bool(((o >= lo - 1e-5) & (o <= hi + 1e-5)).all())


def test_scan_one_stream_of_4096_tiles():
    """A single stream of 2^20 rows: 4096 tiles chained by look-back, the
    longest carry chain any workload has; bitwise repeatable over 100 calls."""
    announce("scan 4096-tile chain")
    B, H, N, d = 1, 1, 1 << 20, 64
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=14, device=dev())
    ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev())
    first = aaren.aaren_scan(q, k, v, workspace=ws)
    for _ in range(99):
        again = aaren.aaren_scan(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(first, again)
    assert scan_header_error(ws) == 0
    ref = oracle.scan(host32(q), host32(k), host32(v), workloads.default_scale(d))
    check(first, ref, 1e-5, "4096-tile chain")
