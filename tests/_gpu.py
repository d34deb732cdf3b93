"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle

# Tolerances on max |o_gpu - o_ref| / (1 + |o_ref|): fp32 inputs 1e-5, bf16
# inputs (fp32 accumulation, any output dtype) 2e-3.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}

# A bfloat16 OUTPUT carries 8 significant bits: rounding alone moves o by up to
# 2^-8 |o| (half an ulp at the bottom of a binade), which exceeds 2e-3 (1 + |o|)
# for |o| near 2. Its bound is that rounding plus the fp32 accumulation slack.
TOL_BF16_OUT = 2.0 ** -8 + 1e-4


def dev():
    return torch.device("cuda:0")


def host32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 host copy (bfloat16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def announce(msg: str):
    """Name the case before a GPU step, flushed, so a failing run says which."""
    print(f"[gpu case] {msg}", file=sys.stderr, flush=True)


def check(got: torch.Tensor, ref: np.ndarray, tol: float, what: str):
    torch.cuda.synchronize()
    err = oracle.max_scaled_err(host32(got), ref)
    assert err <= tol, f"{what}: max scaled error {err:.3e} > {tol:.1e}"
    return err


def scan_header_error(ws: torch.Tensor) -> int:
    """The workspace's error word (0 unless a tile gave up waiting)."""
    return int(ws[12:16].view(torch.int32).item())


# dq = scale * sum_i ds_i k_i adds n = B*N (or T) terms per head. Rounding
# errors of independent signs grow a sum's error like sqrt(n) 2^-24 times the
# terms' size; the tolerance on the scaled error |dq - ref| / (1 + |ref|) is
# 8 sqrt(n) 2^-24, and never below 1e-4. Measured at full size: the dense
# batch (n = 131072, bound 1.7e-4) about 1e-6..4e-6, the packed batch
# (n = 4,151,461, bound 9.8e-4) 1.0e-4. Losing one lane group's 8-row partial
# at the dense shape moves dq by about 6e-3 of (1 + |dq|), which the check
# catches (test_gpu_workloads plants it).
def dq_tol(n_terms: int) -> float:
    return max(1e-4, 8.0 * math.sqrt(n_terms) * 2.0 ** -24)


def gpu_scaled_err(got: torch.Tensor, ref: np.ndarray) -> float:
    """oracle.max_scaled_err, evaluated on the device in float64 (the
    full-size checks compare billions of elements; the host is slow at it).
    Elements NaN on both sides count as equal; any other NaN fails."""
    torch.cuda.synchronize()
    if got.numel() == 0:
        return 0.0
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64)).to(got.device)
    g = got.double()
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {tuple(g.shape)} vs {tuple(r.shape)}")
    err = (g - r).abs_().div_(r.abs().add_(1.0))
    err = torch.where(torch.isnan(g) & torch.isnan(r), torch.zeros_like(err), err)
    if bool(torch.isnan(err).any()):
        return float("inf")
    return float(err.max())


def progress(msg: str):
    """A line per finished part of a long check (flushed)."""
    print(msg, file=sys.stderr, flush=True)
