"""libaaren used from plain C99 (tests/c_client.c): the header and the shared
library with no Python or torch in between. On the CPU the client compiles
(gcc -std=c99 -pedantic, the HIP runtime's C API for device memory) and links
against libaaren.so; on the GPU it runs one aaren_scan and its output is
compared with the CPU oracle's scan of the same inputs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "exact_softmax_attention_02_amd")
ROCM = "/opt/rocm"
B, H, N, D = 2, 3, 600, 64   # as in c_client.c


def _build(tmp_path):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("needs gcc and the ROCm headers")
    if not os.path.exists(os.path.join(PKG, "libaaren.so")):
        pytest.skip("libaaren.so is not built")
    exe = str(tmp_path / "c_client")
    r = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
         "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
         os.path.join(HERE, "c_client.c"), "-o", exe, "-L", PKG, "-laaren",
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib")],
        capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_compiles_and_links(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_client_scan_matches_oracle(tmp_path):
    exe = _build(tmp_path)
    out = str(tmp_path / "scan.f32")
    r = subprocess.run([exe, out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    data = np.fromfile(out, dtype="<f4")
    nq, nk = H * D, B * H * N * D
    assert data.size == nq + 3 * nk
    q = data[:nq].reshape(H, D)
    k = data[nq:nq + nk].reshape(B, H, N, D)
    v = data[nq + nk:nq + 2 * nk].reshape(B, H, N, D)
    o = data[nq + 2 * nk:].reshape(B, H, N, D)
    ref = oracle.scan(q, k, v, 0.125)
    err = oracle.max_scaled_err(o, ref)
    print(f"C client: {r.stdout.strip()}; max scaled err {err:.2e}")
    assert err <= 1e-5, err


def test_header_matches_the_stated_prototypes(tmp_path):
    """tests/abi_contract.c re-declares the boundary's entry points with the
    prototypes the scope table states; C rejects a second declaration of a
    different type, so this compiles only if the header agrees with them."""
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    r = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
         "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_contract.c")],
        capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
