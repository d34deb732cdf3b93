"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

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
