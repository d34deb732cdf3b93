"""bench.py's host side (no GPU): the one-GPU refusal, the workload list, the
source hash that decides whether committed counters still describe the
kernels, and the input checksums."""
import os
import subprocess
import sys

import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr


def test_help_lists_every_workload():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("dense", "long_bf16", "ragged", "stream", "append", "reduce", "backward",
              "self_attn", "layer", "mean_query", "copy"):
        assert w in r.stdout, w


def test_code_only_ignores_comments_and_layout_but_not_code():
    a = "int f(int x) {  // doubles x\n    return 2 * x; /* the\n factor */ }\n"
    b = "int f(int x)\n{\n    return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }\n"
    s = 'const char *s = "// not a comment";\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert "// not a comment" in bench._code_only(s)


def test_source_hash_covers_every_kernel_kind():
    hashes = {kind: bench.source_hash(kind) for kind in bench.KERNEL_SOURCES}
    assert all(len(h) == 64 for h in hashes.values())
    assert bench.source_hash("scan") == bench.source_hash("scan")   # stable


def test_input_checksums_are_exact_word_sums():
    """The sum of the raw words as signed integers, modulo 2^64, in hex: for
    fp32 1.0 (0x3f800000) and -2.0 (0xc0000000 = -2^30), and for the bf16
    halves of the same values (0x3f80 and 0xc000 = -16384)."""
    x = torch.tensor([1.0, -2.0], dtype=torch.float32)
    got = bench.input_checksums({"x": x, "y": x.to(torch.bfloat16), "both": [x, x]})
    assert got["x"] == f"{(0x3f800000 - (1 << 30)) % (1 << 64):016x}"
    assert got["y"] == f"{(0x3f80 - 16384) % (1 << 64):016x}"
    assert got["both"] == f"{(2 * (0x3f800000 - (1 << 30))) % (1 << 64):016x}"
