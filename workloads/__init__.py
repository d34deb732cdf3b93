"""Seeded synthetic inputs for single-query softmax attention.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic: the oracle, the tests, the smoke check and the benchmark
all take their inputs from here, so that the GPU library and the CPU oracle see
the same bytes.

Recipe (every workload is i.i.d. and unstructured; the pages measure the method
on task datasets that are not reproduced here, and these seeded inputs stand in
for them):

* dense:     q [H,d], K,V [B,H,N,d], all N(0,1), drawn in that order from one
             torch.Generator seeded with the workload's seed, on the target device.
* long bf16: as dense, then per (b,h) the keys are multiplied by a factor that
             makes the largest |scale * <q_h, k_i>| equal a given span (80), then
             q, K, V are rounded to bfloat16 (round-to-nearest-even). The factor
             is found with one matmul; it only shapes the input.
* ragged:    sequence lengths uniform in [1, max_len] from numpy's
             default_rng(seed); K,V packed token-major [T,H,d], N(0,1).
* stream:    q [H,d]; per append t, k_t and v_t [S,H,d] N(0,1).
* reduce:    as dense with B = H = 1.
* gradients: the forward's inputs as above; the output gradient dO is N(0,1)
             from its own generator (seed + 100), rounded to bfloat16 for
             bf16 inputs.

The GPU draws (torch's Philox generator) differ from CPU draws for the same
seed; a test always draws on one device and copies the exact bytes to the
other.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One named workload: its kind, sizes, dtype and seed."""
    name: str
    kind: str            # dense | segmented | step | append | self_attention | layer | reduce
    sizes: dict = field(default_factory=dict)
    dtype: str = "f32"   # input dtype: "f32" or "bf16"
    seed: int = 0
    score_span: float | None = None

    def describe(self) -> str:
        s = ", ".join(f"{k}={v}" for k, v in self.sizes.items())
        extra = f", scores span +-{self.score_span:g}" if self.score_span else ""
        return f"{self.kind} {s}, {self.dtype}{extra}, seed {self.seed}"


WORKLOADS = {
    # one sequence, one head: the small case the oracle finishes at once
    "single": Workload("single", "dense", dict(B=1, H=1, N=1024, d=64), "f32", 1),
    # the dense batch the headline throughput is quoted on
    "dense": Workload("dense", "dense", dict(B=32, H=8, N=4096, d=64), "f32", 2),
    # one GPU's share of the dense batch split over 8 GPUs by batch row
    "dense_share": Workload("dense_share", "dense", dict(B=4, H=8, N=4096, d=64), "f32", 2),
    # long sequences, bf16 inputs, scores stretched to +-80
    "long_bf16": Workload("long_bf16", "dense", dict(B=4, H=16, N=65536, d=128), "bf16", 3,
                          score_span=80.0),
    # gradients of the dense batch with bf16 q, K, V and output gradients
    # (the forward's output and log-normaliser stay float32)
    "backward_bf16": Workload("backward_bf16", "dense", dict(B=32, H=8, N=4096, d=64), "bf16", 2),
    # packed variable-length batch
    "ragged": Workload("ragged", "segmented", dict(num_seqs=4096, max_len=8192, H=8, d=64),
                       "f32", 4),
    # gradients of a packed batch a quarter the size of the ragged one (the
    # six gradient-pass tensors of the full one would need ~210 GB)
    "ragged_backward": Workload("ragged_backward", "segmented",
                                dict(num_seqs=1024, max_len=8192, H=8, d=64), "f32", 10),
    # many independent streams, one token appended per call
    "stream": Workload("stream", "step", dict(S=262144, H=4, d=64, steps=256), "f32", 5),
    # the same streams and tokens, 16 tokens appended per call
    "append": Workload("append", "append", dict(S=262144, H=4, d=64, steps=256, block=16), "f32",
                       5),
    # self-attention, one query per token, causal, at the pages' sequence length
    "self_attn": Workload("self_attn", "self_attention", dict(B=2, H=16, N=16384, d=128, causal=1),
                          "bf16", 7),
    # stacked Aaren layers: bf16 projections (rocBLAS) + scan, Dm = H*d
    "layer": Workload("layer", "layer", dict(B=8, N=4096, Dm=1024, H=16, d=64, layers=4), "bf16", 8),
    # global-aggregation attention: each (b,h)'s mean query over its 65536 pairs
    "mean_query": Workload("mean_query", "mean_query", dict(B=4, H=8, N=65536, d=128), "f32", 9),
    # one query over 2^20 keys
    "reduce": Workload("reduce", "reduce", dict(B=1, H=1, N=1 << 20, d=128), "f32", 6),
}


def default_scale(d: int) -> float:
    """The 1/sqrt(d) score scale, rounded once to float32 (the value every
    caller passes, and the value the oracle reads back exactly)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def dense_inputs(B, H, N, d, seed, device="cpu", dtype="f32", score_span=None, scale=None):
    """q [H,d], K,V [B,H,N,d]. With score_span, K is stretched per (b,h) so that
    the largest |scale*<q_h,k_i>| equals score_span before rounding to dtype."""
    g = _gen(seed, device)
    q = torch.randn(H, d, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    td = _torch_dtype(dtype)
    q = q.to(td)
    if score_span is not None and N > 0:
        sc = default_scale(d) if scale is None else scale
        # raw scores of the unscaled keys against the (already rounded) query
        raw = torch.matmul(k, q.float().unsqueeze(-1)).squeeze(-1) * sc    # [B,H,N]
        peak = raw.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)       # [B,H,1]
        k = k * (score_span / peak).unsqueeze(-1)
        del raw
    return q.contiguous(), k.to(td).contiguous(), v.to(td).contiguous()


def segment_lengths(num_seqs: int, max_len: int, seed: int) -> np.ndarray:
    """Lengths uniform on the integers 1..max_len inclusive (numpy default_rng)."""
    rng = np.random.default_rng(seed)
    return rng.integers(1, max_len + 1, size=num_seqs, dtype=np.int64)


def offsets_of(lengths) -> np.ndarray:
    """Exclusive running total of the lengths: offsets[0] = 0, offsets[S] = T."""
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    return out


def segmented_inputs(lengths, H, d, seed, device="cpu", dtype="f32"):
    """q [H,d]; K,V packed token-major [T,H,d]; offsets int64 [S+1] (on device)."""
    offs = offsets_of(lengths)
    T = int(offs[-1])
    g = _gen(seed, device)
    q = torch.randn(H, d, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(T, H, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(T, H, d, generator=g, device=device, dtype=torch.float32)
    td = _torch_dtype(dtype)
    return (q.to(td).contiguous(), k.to(td).contiguous(), v.to(td).contiguous(),
            torch.from_numpy(offs).to(device))


def step_inputs(S, H, d, steps, seed, device="cpu", dtype="f32"):
    """q [H,d]; K_t, V_t [steps,S,H,d] (row t is the token appended by call t)."""
    g = _gen(seed, device)
    q = torch.randn(H, d, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(steps, S, H, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(steps, S, H, d, generator=g, device=device, dtype=torch.float32)
    td = _torch_dtype(dtype)
    return q.to(td).contiguous(), k.to(td).contiguous(), v.to(td).contiguous()


def self_attention_inputs(B, H, N, d, seed, device="cpu", dtype="bf16"):
    """Q, K, V [B,H,N,d] N(0,1), one query per token."""
    g = _gen(seed, device)
    q = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    td = _torch_dtype(dtype)
    return q.to(td).contiguous(), k.to(td).contiguous(), v.to(td).contiguous()


def layer_inputs(B, N, Dm, H, d, layers, seed, device="cpu"):
    """x [B,N,Dm] bf16 N(0,1); per layer w_kv [Dm_l, 2*H*d] bf16 N(0, 1/Dm_l)
    (Dm_l = Dm for the first layer, H*d after) and q [H,d] float32 N(0,1)."""
    g = _gen(seed, device)
    x = torch.randn(B, N, Dm, generator=g, device=device).to(torch.bfloat16)
    ws, qs = [], []
    for layer in range(layers):
        dm = Dm if layer == 0 else H * d
        ws.append((torch.randn(dm, 2 * H * d, generator=g, device=device) / dm ** 0.5)
                  .to(torch.bfloat16))
        qs.append(torch.randn(H, d, generator=g, device=device))
    return x, ws, qs


def mean_query_inputs(B, H, N, d, seed, device="cpu", dtype="f32"):
    """hq, K, V [B,H,N,d]: hq N(0.5, 1) (so the mean query is of order 0.5
    and the weights are not all equal), K and V N(0,1)."""
    g = _gen(seed, device)
    hq = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32) + 0.5
    k = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, device=device, dtype=torch.float32)
    td = _torch_dtype(dtype)
    return hq.to(td).contiguous(), k.to(td).contiguous(), v.to(td).contiguous()


def reduce_inputs(B, H, N, d, seed, device="cpu", dtype="f32"):
    """q [H,d], K,V [B,H,N,d] N(0,1)."""
    return dense_inputs(B, H, N, d, seed, device=device, dtype=dtype)
