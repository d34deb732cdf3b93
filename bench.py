#!/usr/bin/env python3
"""Throughput of libaaren on one MI355X, against the HBM roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the hot path over one batch of the workload, inputs
already resident in HBM:
  dense, single, long_bf16 : one aaren_scan call          (token-heads = B*H*N)
  dense_share              : the dense batch's share of one GPU out of 8 (B=4)
  ragged                   : one aaren_scan_segmented call (token-heads = H*T)
  stream                   : aaren_state_init + 256 aaren_step calls
                                                           (token-heads = S*H*256)
  stream_hbm               : the same 256 calls over 8 state sets in turn, so
                             each call reads its state from HBM (the single
                             set stays mostly in the Infinity Cache)
  append                   : aaren_state_init + 16 aaren_append calls of 16
                             tokens, the same 256 tokens per stream
  backward                 : one aaren_scan_backward call on the dense batch
  backward_bf16            : the same with bf16 q, K, V and output gradients
  ragged_backward          : one aaren_scan_segmented_backward call on a packed
                             batch of 1024 sequences
  mean_query               : one aaren_mean_query_attention call (keys/s)
  layer                    : 4 stacked aaren_layer_forward calls (rocBLAS
                             projections + scan; tokens = B*N through all)
  self_attn                : one aaren_self_attention call (causal, one query
                             per token; matrix cores: TFLOP/s against the bf16
                             peak)
  reduce                   : one aaren_reduce call         (keys = B*H*N)
W untimed steps, then exactly K steps between two HIP events recorded on the
stream the kernels run on. Prints one JSON line. The default workload is the
dense batch (B=32, H=8, N=4096, d=64, fp32) the headline metric is quoted on.

roofline.achieved = algorithmic bytes per launch of the dominant kernel /
its average duration over the timed region; algorithmic bytes = K and V read
once and O written once (plus the state for the step). roofline.traffic is the
HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled
by the same counters on a plain copy of known size), read from the committed
counter file under profiles/ only while the kernel sources still hash to the
value recorded there; otherwise null.

cpu_baseline times the float64 CPU oracle (as it is, untuned) on the host's
cores over a bounded sample of the same workload; for the dense workload it
adds the same oracle on one thread (cpu_baseline.one_thread); the single
sequence is one unit and runs on one thread anyway.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD's published figure
# Steps rotate over enough copies of the inputs and outputs that one pass over
# them moves at least this many bytes: eight times the 256 MB Infinity Cache,
# so a step's data comes from HBM and not from what the previous step left in
# the cache.
ROTATE_BYTES = 2 << 30
MAX_SETS = 8


def n_sets(bytes_per_step: int) -> int:
    return max(1, min(MAX_SETS, -(-ROTATE_BYTES // bytes_per_step)))
KERNEL_SOURCES = {
    "scan": ["scan.hip", "scan_tiles.h", "lookback.h", "device.h", "layout.h"],
    "backward": ["scan_backward.hip", "lookback.h", "device.h", "layout.h"],
    "step": ["step.hip", "device.h", "layout.h"],
    "append": ["step.hip", "device.h", "layout.h"],
    "self_attention": ["self_attention.hip", "self_attention.h", "device.h", "layout.h"],
    "layer": ["layer.hip", "scan.hip", "scan_tiles.h", "lookback.h", "device.h", "layout.h"],
    "reduce": ["reduce.hip", "device.h", "layout.h"],
    "mean_query": ["reduce.hip", "device.h", "layout.h"],
}


def _code_only(text: str) -> str:
    """C++ source without comments, whitespace runs collapsed: what decides
    the compiled kernel (string and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(kind: str) -> str:
    """Hash of the code (comments and layout ignored) of a kernel kind's sources:
    counters taken from other code are not reported as this code's traffic."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "exact_softmax_attention_02_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter file, or None
    if there is none or the kernel changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha256") != source_hash(kind):
        return None
    return (c["fetch_kib_per_dispatch"] * 1024 * c["copy_fetch_factor"] +
            c["write_kib_per_dispatch"] * 1024 * c["copy_write_factor"])


def input_checksums(inputs) -> dict:
    """Per input tensor (or list of tensors): the sum of its raw words as signed
    integers (32-bit words for fp32, 16-bit for bf16, 64-bit for int64), taken
    on the device in int64 and reported modulo 2^64 in hex. Exact and order-free,
    so it identifies the bytes a run used without copying them to the host."""
    import torch
    words = {8: torch.int64, 4: torch.int32, 2: torch.int16, 1: torch.int8}
    out = {}
    for name, t in inputs.items():
        total = 0
        for x in (t if isinstance(t, (list, tuple)) else [t]):
            total += int(x.contiguous().view(words[x.element_size()]).sum(dtype=torch.int64))
        out[name] = f"{total % (1 << 64):016x}"
    return out


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Workload:
    """A prepared workload: step() runs one pass; the numbers describe it."""
    kind = "scan"
    unit = "token-heads/s"
    launches_per_step = 1
    sets = 1


def make(name: str, device):
    import numpy as np
    import torch

    import exact_softmax_attention_02_amd as aaren
    import workloads as wl

    b = Workload()
    b.name = name
    if name != "copy":
        w = wl.WORKLOADS[{"backward": "dense", "stream_hbm": "stream"}.get(name, name)]
        z = w.sizes
        b.describe = w.describe()
        b.dtype = {"f32": "f32", "bf16": "bf16->f32"}[w.dtype]

    if name == "copy":
        # a plain device copy of known size (the dense batch's K): the practical
        # read+write ceiling, and the reference the HBM counters are scaled by
        # no input checksum here: its small device-to-host copy would run as a
        # copy kernel too and blur this calibration
        x = torch.randn(32, 8, 4096, 64, device=device)
        b.sets = n_sets(2 * x.numel() * 4)
        bufs = [(x, torch.empty_like(x))] + [(x.clone(), torch.empty_like(x))
                                             for _ in range(b.sets - 1)]
        turn = [0]

        def step():
            src, dst = bufs[turn[0] % b.sets]
            turn[0] += 1
            dst.copy_(src)
        b.step = step
        b.kind = "copy"
        b.unit = "bytes/s"
        b.units = 2 * x.numel() * 4
        b.bytes_per_launch = 2 * x.numel() * 4
        b.config = {"workload": "plain device copy, 268,435,456 B read + 268,435,456 B written"}
        b.kernel = "torch elementwise copy"
        b.dtype = "f32"
        b.describe = "copy"
        b.cpu = None
        return b

    if name in ("backward", "backward_bf16"):
        # gradients of the dense batch: the forward's o and lse are inputs;
        # bf16: q, k, v and the output gradient in bf16, o and lse float32
        B, H, N, d = z["B"], z["H"], z["N"], z["d"]
        q, k, v = wl.dense_inputs(B, H, N, d, w.seed, device=device, dtype=w.dtype)
        scale = wl.default_scale(d)
        o, lse = aaren.aaren_scan(q, k, v, scale, return_lse=True)
        g = torch.randn(B, H, N, d, device=device,
                        generator=torch.Generator(device=device).manual_seed(w.seed + 100))
        g = g.to(k.dtype)
        b.inputs = dict(q=q, k=k, v=v, dout=g)
        dq = torch.empty(H, d, device=device)
        ws = torch.zeros(aaren.aaren_scan_backward_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device=device)
        # k, v, dout in their dtype; o read and dk, dv written in float32
        b.bytes_per_launch = (3 * k.numel() * k.element_size() + 3 * k.numel() * 4 +
                              lse.numel() * 4 + dq.numel() * 4)
        b.sets = n_sets(b.bytes_per_launch)
        f32 = torch.float32
        bufs = [(k, v, o, g, lse, torch.empty_like(k, dtype=f32), torch.empty_like(v, dtype=f32))]
        bufs += [tuple(x.clone() for x in bufs[0][:5]) +
                 (torch.empty_like(k, dtype=f32), torch.empty_like(v, dtype=f32))
                 for _ in range(b.sets - 1)]
        turn = [0]

        def step():
            kk, vv, oo, gg, ll, dk, dv = bufs[turn[0] % b.sets]
            turn[0] += 1
            aaren.aaren_scan_backward(q, kk, vv, oo, gg, ll, scale, dq=dq, dk=dk, dv=dv,
                                      workspace=ws)
        b.step = step
        b.kind = "backward"
        b.units = B * H * N
        b.launches_per_step = 1
        b.config = {"workload": f"gradients of the dense many-to-many scan {b.describe}", "B": B,
                    "H": H, "N": N, "d": d, "in_dtype": w.dtype, "out_dtype": "f32"}
        b.kernel = "scan_backward_kernel + scan_backward_dq_kernel"

        def cpu(budget_s):
            import oracle
            qh, kh, vh, gh = (t.float().cpu().numpy() for t in (q, k, v, g))
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.scan_backward(qh, kh, vh, gh, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * B * H * N / dt, f"{done} pass(es) over {B}x{H}x{N} (d={d}) gradients"
        b.cpu = cpu
        return b

    if name == "ragged_backward":
        H, d = z["H"], z["d"]
        lengths = wl.segment_lengths(z["num_seqs"], z["max_len"], w.seed)
        q, k, v, offs = wl.segmented_inputs(lengths, H, d, w.seed, device=device)
        T = int(lengths.sum())
        scale = wl.default_scale(d)
        o, lse = aaren.aaren_scan_segmented(q, k, v, offs, scale, return_lse=True)
        g = torch.randn(T, H, d, device=device,
                        generator=torch.Generator(device=device).manual_seed(w.seed + 100))
        b.inputs = dict(q=q, k=k, v=v, offsets=offs, dout=g)
        dq, dk, dv = torch.empty(H, d, device=device), torch.empty_like(k), torch.empty_like(v)
        ws = torch.zeros(aaren.aaren_scan_segmented_backward_workspace_size(len(lengths), T, H, d),
                         dtype=torch.uint8, device=device)
        b.step = lambda: aaren.aaren_scan_segmented_backward(q, k, v, o, g, lse, offs, scale, dq=dq,
                                                             dk=dk, dv=dv, workspace=ws)
        b.kind = "backward"
        b.units = H * T
        b.bytes_per_launch = 6 * T * H * d * 4 + T * H * 4 + offs.numel() * 8 + H * d * 4
        b.config = {"workload": f"gradients of the packed many-to-many scan {b.describe}",
                    "num_seqs": len(lengths), "total_tokens": T, "H": H, "d": d,
                    "in_dtype": "f32", "out_dtype": "f32"}
        b.kernel = "scan_backward_kernel (packed) + scan_backward_dq_kernel"

        def cpu(budget_s):
            import oracle
            ho = offs.cpu().numpy()
            n = 1
            while n < len(lengths) and ho[n] < 500_000:
                n += 1
            qh = q.cpu().numpy()
            kh, vh, gh = (t[:ho[n]].cpu().numpy() for t in (k, v, g))
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.scan_segmented_backward(qh, kh, vh, gh, ho[:n + 1], scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * H * int(ho[n]) / dt, (f"{done} pass(es) over the first {n} sequences "
                                                 f"({int(ho[n])} tokens x {H} heads)")
        b.cpu = cpu
        return b

    if w.kind == "dense":
        B, H, N, d = z["B"], z["H"], z["N"], z["d"]
        q, k, v = wl.dense_inputs(B, H, N, d, w.seed, device=device, dtype=w.dtype,
                                  score_span=w.score_span)
        b.inputs = dict(q=q, k=k, v=v)
        scale = wl.default_scale(d)
        o = torch.empty(B, H, N, d, device=device)
        ws = torch.zeros(aaren.aaren_scan_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device=device)
        b.bytes_per_launch = 2 * k.numel() * k.element_size() + o.numel() * 4
        b.sets = n_sets(b.bytes_per_launch)
        bufs = [(k, v, o)] + [(k.clone(), v.clone(), torch.empty_like(o))
                              for _ in range(b.sets - 1)]
        turn = [0]

        def step():
            kk, vv, oo = bufs[turn[0] % b.sets]
            turn[0] += 1
            aaren.aaren_scan(q, kk, vv, scale, out=oo, workspace=ws)
        b.step = step
        b.units = B * H * N
        b.config = {"workload": f"dense many-to-many scan {b.describe}", "B": B, "H": H, "N": N,
                    "d": d, "in_dtype": w.dtype, "out_dtype": "f32"}
        b.kernel = "scan_kernel"

        def cpu(budget_s):
            import oracle
            qh, kh, vh = (t.float().cpu().numpy() for t in (q, k, v))
            rows = B if name != "long_bf16" else 1      # long_bf16: one batch row
            kh, vh = kh[:rows], vh[:rows]
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.scan(qh, kh, vh, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return (done * rows * H * N / dt,
                    f"{done} pass(es) over {rows}x{H}x{N} (d={d}) of the workload's inputs")
        b.cpu = cpu

    elif w.kind == "segmented":
        H, d = z["H"], z["d"]
        lengths = wl.segment_lengths(z["num_seqs"], z["max_len"], w.seed)
        q, k, v, offs = wl.segmented_inputs(lengths, H, d, w.seed, device=device)
        b.inputs = dict(q=q, k=k, v=v, offsets=offs)
        T = int(lengths.sum())
        scale = wl.default_scale(d)
        o = torch.empty(T, H, d, device=device)
        ws = torch.zeros(aaren.aaren_scan_segmented_workspace_size(len(lengths), T, H, d),
                         dtype=torch.uint8, device=device)
        b.step = lambda: aaren.aaren_scan_segmented(q, k, v, offs, scale, out=o, workspace=ws)
        b.units = H * T
        b.bytes_per_launch = 3 * T * H * d * 4 + offs.numel() * 8
        b.config = {"workload": f"packed ragged many-to-many scan {b.describe}",
                    "num_seqs": len(lengths), "total_tokens": T, "H": H, "d": d,
                    "in_dtype": "f32", "out_dtype": "f32"}
        b.kernel = "scan_kernel (segmented)"

        def cpu(budget_s):
            import oracle
            ho = offs.cpu().numpy()
            qh = q.cpu().numpy()
            n = 1
            while n < len(lengths) and ho[n] < 2_000_000:
                n += 1
            kh, vh = k[:ho[n]].cpu().numpy(), v[:ho[n]].cpu().numpy()
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.scan_segmented(qh, kh, vh, ho[:n + 1], scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * H * int(ho[n]) / dt, (f"{done} pass(es) over the first {n} sequences "
                                                 f"({int(ho[n])} tokens x {H} heads)")
        b.cpu = cpu

    elif w.kind == "step":
        S, H, d, T = z["S"], z["H"], z["d"], z["steps"]
        q, k, v = wl.step_inputs(S, H, d, T, w.seed, device=device)
        b.inputs = dict(q=q, k=k, v=v)
        scale = wl.default_scale(d)
        # stream_hbm: the same calls over 8 state sets in turn (each set takes
        # every 8th token), so that a call's state was last touched 7 calls
        # (about 9.5 GB of traffic) earlier and comes from HBM, not from the
        # 256 MB Infinity Cache the single state set mostly stays in
        nstate = 8 if name == "stream_hbm" else 1
        states = [aaren.new_state(S, H, d, device=device) for _ in range(nstate)]
        m, u, st_w = states[0]
        o = torch.empty(S, H, d, device=device)

        # events every T/8 appends (the last step's are kept): the time per
        # append must not grow with t, the state being constant-size
        seg = max(1, T // 8)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(T // seg + 1)]
        stream_ = torch.cuda.current_stream(device)

        def step():
            for sm, su, sw in states:
                aaren.aaren_state_init(sm, su, sw)
            for t in range(T):
                if t % seg == 0:
                    marks[t // seg].record(stream_)
                sm, su, sw = states[t % nstate]
                aaren.aaren_step(q, k[t], v[t], sm, su, sw, scale, o_t=o)
            if T % seg == 0:
                marks[-1].record(stream_)

        def per_append_by_segment():
            torch.cuda.synchronize()
            return [round(marks[i].elapsed_time(marks[i + 1]) * 1e3 / seg, 2)
                    for i in range(len(marks) - 1)]
        b.extra = lambda: {"us_per_append_by_eighth": per_append_by_segment()}
        b.step = step
        b.kind = "step"
        b.units = S * H * T
        b.launches_per_step = T
        # per stream-head and append: k, v, w read; w, o written (5 x d x 4 B);
        # m, u read and written (16 B)
        b.bytes_per_launch = S * H * (5 * d * 4 + 4 * 4)
        b.config = {"workload": f"RNN step, {T} appends per stream {b.describe}", "S": S, "H": H,
                    "d": d, "appends": T, "in_dtype": "f32", "out_dtype": "f32",
                    "state_sets": nstate}
        if nstate > 1:
            b.config["workload"] = (f"RNN step, {T} calls over {nstate} state sets in turn "
                                    f"({T // nstate} appends each; state read from HBM) "
                                    f"{b.describe}")
        b.kernel = "step_kernel"

        def cpu(budget_s):
            import oracle
            ns = 4096
            qh, kh, vh = q.cpu().numpy(), k[:, :ns].cpu().numpy(), v[:, :ns].cpu().numpy()
            done, t0 = 0, time.perf_counter()
            while True:
                st = oracle.state_init(ns, H, d)
                for t in range(T):
                    oracle.step(qh, kh[t], vh[t], st, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * ns * H * T / dt, f"{done} pass(es) over {ns} streams x {H} heads x {T} appends"
        b.cpu = cpu

    elif w.kind == "append":
        S, H, d, T, blk = z["S"], z["H"], z["d"], z["steps"], z["block"]
        q, k, v = wl.step_inputs(S, H, d, T, w.seed, device=device)
        b.inputs = dict(q=q, k=k, v=v)
        scale = wl.default_scale(d)
        m, u, st_w = aaren.new_state(S, H, d, device=device)
        o = torch.empty(blk, S, H, d, device=device)

        def step():
            aaren.aaren_state_init(m, u, st_w)
            for t0 in range(0, T, blk):
                aaren.aaren_append(q, k[t0:t0 + blk], v[t0:t0 + blk], m, u, st_w, scale, o=o)
        b.step = step
        b.kind = "append"
        b.units = S * H * T
        b.launches_per_step = T // blk
        # per stream-head and call: blk x (k, v read, o written) rows of d x 4 B,
        # plus the state (w, m, u) read and written once
        b.bytes_per_launch = S * H * (blk * 3 * d * 4 + 2 * (d * 4 + 8))
        b.config = {"workload": f"multi-token append, {T} tokens per stream in {T // blk} calls of "
                                f"{blk} {b.describe}", "S": S, "H": H, "d": d, "tokens": T,
                    "tokens_per_call": blk, "in_dtype": "f32", "out_dtype": "f32"}
        b.kernel = "append_kernel"

        def cpu(budget_s):
            import oracle
            ns = 4096
            qh, kh, vh = q.cpu().numpy(), k[:, :ns].cpu().numpy(), v[:, :ns].cpu().numpy()
            done, t0 = 0, time.perf_counter()
            while True:
                st = oracle.state_init(ns, H, d)
                for a in range(0, T, blk):
                    oracle.append(qh, kh[a:a + blk], vh[a:a + blk], st, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * ns * H * T / dt, (f"{done} pass(es) over {ns} streams x {H} heads x {T} "
                                             f"tokens in appends of {blk}")
        b.cpu = cpu

    elif w.kind == "self_attention":
        B, H, N, d, causal = z["B"], z["H"], z["N"], z["d"], bool(z["causal"])
        q, k, v = wl.self_attention_inputs(B, H, N, d, w.seed, device=device)
        b.inputs = dict(q=q, k=k, v=v)
        scale = wl.default_scale(d)
        o = torch.empty(B, H, N, d, device=device)
        ws = torch.empty(aaren.aaren_self_attention_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device=device)
        b.step = lambda: aaren.aaren_self_attention(q, k, v, scale, causal=causal, out=o,
                                                    workspace=ws)
        b.kind = "self_attention"
        b.unit = "TFLOP/s"
        b.bound = "mfma"
        # algorithmic flops: 2d for q.k and 2d for p.v per (query, key) pair
        pairs = N * (N + 1) // 2 if causal else N * N
        b.flops_per_launch = 4 * d * pairs * B * H
        b.units = b.flops_per_launch / 1e12
        b.bytes_per_launch = 3 * q.numel() * 2 + o.numel() * 4
        b.config = {"workload": f"self-attention, one query per token {b.describe}", "B": B, "H": H,
                    "N": N, "d": d, "causal": causal, "in_dtype": "bf16", "out_dtype": "f32",
                    "flops_per_call": b.flops_per_launch}
        b.kernel = "self_attention_kernel (+ attn_vmax_kernel, attn_transpose_kernel)"

        def cpu(budget_s):
            import oracle
            rows = 256
            qh, kh, vh = (t[:1, :1].float().cpu().numpy() for t in (q, k, v))
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.self_attention(qh, kh, vh, scale, causal=causal, rows=(N - rows, N))
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            per = sum(4 * d * ((i + 1) if causal else N) for i in range(N - rows, N))
            return done * per / dt / 1e12, (f"{done} pass(es) over the last {rows} query rows of "
                                            f"one head (N={N}, d={d})")
        b.cpu = cpu

    elif w.kind == "mean_query":
        B, H, N, d = z["B"], z["H"], z["N"], z["d"]
        hq, k, v = wl.mean_query_inputs(B, H, N, d, w.seed, device=device)
        b.inputs = dict(hq=hq, k=k, v=v)
        scale = wl.default_scale(d)
        o = torch.empty(B, H, d, device=device)
        ws = torch.empty(aaren.aaren_mean_query_attention_workspace_size(B, H, N, d),
                         dtype=torch.uint8, device=device)
        b.bytes_per_launch = 3 * k.numel() * 4 + o.numel() * 4
        b.sets = n_sets(b.bytes_per_launch)
        bufs = [(hq, k, v)] + [(hq.clone(), k.clone(), v.clone()) for _ in range(b.sets - 1)]
        turn = [0]

        def step():
            hh, kk, vv = bufs[turn[0] % b.sets]
            turn[0] += 1
            aaren.aaren_mean_query_attention(hh, kk, vv, scale, out=o, workspace=ws)
        b.step = step
        b.kind = "mean_query"
        b.unit = "keys/s"
        b.units = B * H * N
        b.config = {"workload": f"mean-query attention {b.describe}", "B": B, "H": H, "N": N,
                    "d": d, "in_dtype": "f32", "out_dtype": "f32"}
        b.kernel = "mean_partial_kernel + mean_final_kernel + reduce kernels"

        def cpu(budget_s):
            import oracle
            hh, kh, vh = (t[:1, :1].cpu().numpy() for t in (hq, k, v))
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.mean_query_attention(hh, kh, vh, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * N / dt, f"{done} pass(es) over one (b,h) of {N} pairs (one unit: 1 thread)"
        b.cpu = cpu

    elif w.kind == "layer":
        B, N, Dm, H, d, L = z["B"], z["N"], z["Dm"], z["H"], z["d"], z["layers"]
        x, ws_, qs = wl.layer_inputs(B, N, Dm, H, d, L, w.seed, device=device)
        b.inputs = dict(x=x, w_kv=ws_, q=qs)
        scale = wl.default_scale(d)
        bufs = [torch.empty(B, N, H, d, dtype=torch.bfloat16, device=device) for _ in range(2)]
        work = torch.zeros(aaren.aaren_layer_workspace_size(B, N, max(Dm, H * d), H, d), dtype=torch.uint8,
                           device=device)

        def step():
            h = x
            for layer in range(L):
                h = aaren.aaren_layer_forward(h.reshape(B, N, -1), ws_[layer], qs[layer], scale,
                                              out=bufs[layer % 2], workspace=work)
        b.step = step
        b.kind = "layer"
        b.unit = "tokens/s"
        b.bound = "mfma"
        # Flops of the folded layer (2 per multiply-add): the product's V columns
        # and one score column per head (u_h = W_K^h q_h; its three-part split
        # and the zero column are not counted), plus the scan's 2d per
        # token-head for the weighted sum of V. K = x W_K is never formed.
        b.flops_per_launch = sum(2 * B * N * (Dm if l == 0 else H * d) * (H * d + H) +
                                 2 * d * B * N * H for l in range(L))
        b.units = B * N
        b.bytes_per_launch = 0
        # the same layers by the definition's count, K = x W_K formed: context only
        flops_with_k = sum(2 * B * N * (Dm if l == 0 else H * d) * 2 * H * d + 4 * d * B * N * H
                           for l in range(L))
        b.config = {"workload": f"{L} stacked Aaren layers {b.describe}", "B": B, "N": N,
                    "Dm": Dm, "H": H, "d": d, "layers": L, "in_dtype": "bf16",
                    "out_dtype": "bf16", "flops_per_step": b.flops_per_launch,
                    "flops_per_step_with_k_formed": flops_with_k}
        b.kernel = "layer_fold_kernel + rocBLAS projection GEMMs + scan_kernel (the whole stack)"
        b.dispatches_per_launch = L  # traffic counters are read per layer (fold, GEMM, scan)

        def cpu(budget_s):
            import oracle
            xh = x[:1].float().cpu().numpy()
            wh, qh = ws_[0].float().cpu().numpy(), qs[0].cpu().numpy()
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.layer_forward(xh, wh, qh, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * N / L / dt, f"{done} pass(es) of the first layer over one batch row of {N} tokens (rate per stack of {L})"
        b.cpu = cpu

    else:  # reduce
        B, H, N, d = z["B"], z["H"], z["N"], z["d"]
        q, k, v = wl.reduce_inputs(B, H, N, d, w.seed, device=device)
        b.inputs = dict(q=q, k=k, v=v)
        scale = wl.default_scale(d)
        o = torch.empty(B, H, d, device=device)
        ws = torch.empty(aaren.aaren_reduce_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device=device)
        b.kind = "reduce"
        b.unit = "keys/s"
        b.units = B * H * N
        b.bytes_per_launch = 2 * k.numel() * 4 + o.numel() * 4
        b.sets = n_sets(b.bytes_per_launch)
        bufs = [(k, v)] + [(k.clone(), v.clone()) for _ in range(b.sets - 1)]
        turn = [0]

        def step():
            kk, vv = bufs[turn[0] % b.sets]
            turn[0] += 1
            aaren.aaren_reduce(q, kk, vv, scale, out=o, workspace=ws)
        b.step = step
        b.config = {"workload": f"many-to-one reduction {b.describe}", "B": B, "H": H, "N": N,
                    "d": d, "in_dtype": "f32", "out_dtype": "f32"}
        b.kernel = "reduce_partial_kernel + reduce_final_kernel"

        def cpu(budget_s):
            import oracle
            qh, kh, vh = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
            done, t0 = 0, time.perf_counter()
            while True:
                oracle.reduce(qh, kh, vh, scale)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            dt = time.perf_counter() - t0
            return done * B * H * N / dt, f"{done} pass(es) over all {N} keys (one unit: 1 thread)"
        b.cpu = cpu
    return b


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense",
                    choices=["single", "dense", "dense_share", "long_bf16", "ragged", "stream",
                             "append",
                             "stream_hbm", "reduce", "backward", "backward_bf16",
                             "ragged_backward",
                             "self_attn", "layer",
                             "mean_query", "copy"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-oracle time budget for cpu_baseline (0 to skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path is data-parallel over independent "
              "sequences, and a run of several GPUs would repeat the same per-GPU work; "
              "--gpus must be 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    device = torch.device("cuda:0")
    b = make(args.workload, device)
    checksums = input_checksums(getattr(b, "inputs", {}))
    stream = torch.cuda.current_stream(device)
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        b.step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    value = b.units / (ms / 1e3)
    launch_s = ms / 1e3 / b.launches_per_step
    achieved = b.bytes_per_launch / launch_s / 1e9
    traffic = measured_traffic(b.kind, args.workload) if b.kind != "copy" else None
    if traffic is not None:
        traffic *= getattr(b, "dispatches_per_launch", 1)  # counters are per kernel dispatch
    if getattr(b, "bound", "hbm") == "mfma":
        tflops = b.flops_per_launch / launch_s / 1e12
        roofline = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                    "kernel": b.kernel, "algorithmic_flops_per_launch": b.flops_per_launch}
    else:
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                    "kernel": b.kernel, "algorithmic_bytes_per_launch": b.bytes_per_launch}

    cpu = None
    if args.cpu_seconds > 0 and b.cpu is not None:
        import oracle
        rate, sample = b.cpu(args.cpu_seconds)
        cores = oracle.threads()
        if args.workload in ("reduce", "mean_query", "single"):
            cores = 1  # one unit: the recurrence runs on one thread
        elif args.workload == "ragged_backward":
            cores = min(cores, b.config["H"])  # each sequence's heads are its parallel units
        cpu = {"value": rate, "unit": b.unit, "cores": cores, "kind": "oracle", "sample": sample,
               "cpu_model": host_cpu(), "host_threads": os.cpu_count()}
        if args.workload == "dense":
            # the same oracle on one thread, for the single-core rate
            oracle.set_threads(1)
            try:
                rate1, sample1 = b.cpu(max(args.cpu_seconds / 2, 1.0))
            finally:
                oracle.set_threads(cores)
            cpu["one_thread"] = {"value": rate1, "unit": b.unit, "sample": sample1}

    line = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak) for aaren_scan at B*H*N, d=64/128"
                  if b.kind == "scan" else f"{b.unit} for {args.workload}",
        "value": value,
        "unit": b.unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic (seeded i.i.d. normal inputs; no dataset)",
        "config": dict(b.config, input_sets=b.sets, input_checksums=checksums,
                       **(b.extra() if getattr(b, "extra", None) else {}),
                       note=("steps rotate over input copies so that each step reads HBM"
                             if b.sets > 1 else "one input set")),
        "achieved_GBps": achieved,
        "peak_frac": achieved / PEAK_HBM_GBS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "platform": {"hip": torch.version.hip, "torch": torch.__version__,
                     "device": torch.cuda.get_device_name(device)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
