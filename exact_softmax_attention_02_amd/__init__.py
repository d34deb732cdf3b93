"""Python binding of libaaren (exact single-query softmax attention, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libaaren.so. torch supplies device memory and the current stream.
The functions carry the names of the C entry points declared in
include/aaren.h; see there for the definitions and the contract.

There is no fallback: if libaaren.so is missing, importing this package
fails.

With AAREN_DEBUG=1 in the environment, every scan and scan gradient call
synchronises afterwards and raises AarenError if its workspace reports that
a workgroup could not take part normally (see aaren_workspace_status).
"""
from __future__ import annotations

# torch must be imported before libaaren.so is loaded, so that the library
# binds to the HIP runtime torch has loaded (one runtime per process).
import torch  # noqa: I001

import ctypes
import functools
import itertools
import math
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaaren.so")

AAREN_OK, AAREN_ERR_INVALID_ARG, AAREN_ERR_UNSUPPORTED = 0, 1, 2
AAREN_ERR_ALIGNMENT, AAREN_ERR_WORKSPACE, AAREN_ERR_HIP = 3, 4, 5
AAREN_F32, AAREN_BF16 = 0, 1

EXPORTS = (
    "aaren_version", "aaren_status_string", "aaren_last_error", "aaren_workspace_clear",
    "aaren_init", "aaren_workspace_status", "aaren_scan_lse", "aaren_scan_segmented_lse",
    "aaren_scan_noalloc",
    "aaren_scan_workspace_size", "aaren_scan", "aaren_scan_segmented_workspace_size",
    "aaren_scan_segmented", "aaren_state_init", "aaren_step", "aaren_reduce_workspace_size",
    "aaren_reduce", "aaren_scan_backward_workspace_size", "aaren_scan_backward", "aaren_append",
    "aaren_self_attention_workspace_size", "aaren_self_attention", "aaren_scan_strided",
    "aaren_layer_workspace_size", "aaren_layer_forward",
    "aaren_mean_query_attention_workspace_size", "aaren_mean_query_attention",
    "aaren_scan_segmented_backward_workspace_size", "aaren_scan_segmented_backward",
)


class AarenError(RuntimeError):
    """A libaaren call returned a non-OK status."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"libaaren status {status}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run "
                          "python exact_softmax_attention_02_amd/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, F, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_int
    sig = {
        "aaren_version": (I, []),
        "aaren_status_string": (ctypes.c_char_p, [I]),
        "aaren_last_error": (ctypes.c_char_p, []),
        "aaren_workspace_clear": (I, [P, SZ, P]),
        "aaren_init": (I, []),
        "aaren_workspace_status": (I, [P, SZ, P, I, P]),
        "aaren_scan_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan": (I, [P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ, P]),
        "aaren_scan_lse": (I, [P, P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ, P]),
        "aaren_scan_noalloc": (I, [P, P, P, P, I64, I64, I64, I64, F, I, I, P]),
        "aaren_scan_segmented_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan_segmented": (I, [P, P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ, P]),
        "aaren_scan_segmented_lse": (I, [P, P, P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ,
                                         P]),
        "aaren_state_init": (I, [P, P, P, I64, I64, I64, P]),
        "aaren_step": (I, [P, P, P, P, P, P, P, I64, I64, I64, F, I, I, P]),
        "aaren_append": (I, [P, P, P, P, P, P, P, I64, I64, I64, I64, F, I, I, P]),
        "aaren_self_attention_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan_strided": (I, [P, P, P, P, P, I64, I64, I64, I64, P, P, F, I, I, P, SZ, P]),
        "aaren_layer_workspace_size": (SZ, [I64, I64, I64, I64, I64]),
        "aaren_mean_query_attention_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan_segmented_backward_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan_segmented_backward": (I, [P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, F,
                                              I, P, SZ, P]),
        "aaren_mean_query_attention": (I, [P, P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ, P]),
        "aaren_layer_forward": (I, [P, P, P, P, I64, I64, I64, I64, I64, F, I, P, SZ, P]),
        "aaren_self_attention": (I, [P, P, P, P, P, I64, I64, I64, I64, F, I, I, I, P, SZ, P]),
        "aaren_reduce_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_reduce": (I, [P, P, P, P, P, P, I64, I64, I64, I64, F, I, I, P, SZ, P]),
        "aaren_scan_backward_workspace_size": (SZ, [I64, I64, I64, I64]),
        "aaren_scan_backward": (I, [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, F, I, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _on_tensor_device(fn):
    """Run a binding with its tensors' GPU as the current device: the library
    launches on the calling thread's current device."""
    @functools.wraps(fn)
    def call(*args, **kwargs):
        for a in itertools.chain(args, kwargs.values()):
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return call


# ---- helpers -----------------------------------------------------------------

def _check(status: int):
    if status != AAREN_OK:
        raise AarenError(status, lib.aaren_last_error().decode(errors="replace"))


_DEBUG = os.environ.get("AAREN_DEBUG", "0") not in ("", "0")


def _debug_check(ws, what: str):
    """With AAREN_DEBUG set: wait for the call and raise if its workspace
    reports a workgroup that could not take part normally."""
    if _DEBUG and ws is not None:
        flags = aaren_workspace_status(ws)
        if flags:
            raise AarenError(AAREN_ERR_HIP, f"{what}: workspace error flags {flags:#x}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return AAREN_F32
    if t == torch.bfloat16:
        return AAREN_BF16
    raise TypeError(f"libaaren takes float32 or bfloat16 tensors, not {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts, strided=()):
    """The device of the given tensors; every tensor must be on one GPU and,
    unless it is one of `strided`, contiguous."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libaaren tensors must be on a GPU")
        if not t.is_contiguous() and not any(t is x for x in strided):
            raise ValueError("libaaren tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("libaaren tensors must share one device")
    return dev


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32."""
    return float(np.float32(1.0 / math.sqrt(d)))


_workspaces: dict = {}


def _workspace(kind: str, nbytes: int, device, zeroed: bool):
    """A cached workspace per (kind, device, stream), grown on demand. Scan
    workspaces are zero-filled when allocated (the library keeps them ready
    afterwards); calls on one stream never overlap, so one buffer per stream
    is enough."""
    if nbytes == 0:
        return None
    key = (kind, device, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        alloc = torch.zeros if zeroed else torch.empty
        ws = alloc(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# ---- entry points ------------------------------------------------------------

_initialised: set = set()


def aaren_init(device=None):
    """Prepare a GPU (the current one by default) for the calls that keep
    library state (the layer's rocBLAS handle). Allocates; not under graph
    capture. Repeated calls do nothing."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    if device in _initialised:
        return
    if torch.cuda.is_current_stream_capturing():
        raise AarenError(AAREN_ERR_UNSUPPORTED,
                         "aaren_init allocates and cannot run under graph capture")
    with torch.cuda.device(device):
        _check(lib.aaren_init())
    _initialised.add(device)


@_on_tensor_device
def aaren_workspace_status(workspace: torch.Tensor, reset: bool = False) -> int:
    """The workspace's error flags (0: every scan that used it ran normally;
    bits 1, 2, 4 as in include/aaren.h); waits for the current stream. With
    reset, the flags are cleared after they are read."""
    dev = _need_cuda(workspace)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(lib.aaren_workspace_status(_ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _ptr(flags), int(bool(reset)), _stream(dev)))
    return int(flags.item()) & 0xFFFFFFFF


def aaren_version() -> int:
    return int(lib.aaren_version())


def aaren_last_error() -> str:
    return lib.aaren_last_error().decode(errors="replace")


def aaren_status_string(status: int) -> str:
    return lib.aaren_status_string(status).decode()


def aaren_scan_workspace_size(B, H, N, d) -> int:
    return int(lib.aaren_scan_workspace_size(B, H, N, d))


def aaren_scan_segmented_workspace_size(num_seqs, total_tokens, H, d) -> int:
    return int(lib.aaren_scan_segmented_workspace_size(num_seqs, total_tokens, H, d))


def aaren_reduce_workspace_size(B, H, N, d) -> int:
    return int(lib.aaren_reduce_workspace_size(B, H, N, d))


@_on_tensor_device
def aaren_workspace_clear(workspace: torch.Tensor):
    """Zero a workspace on the current stream (needed once, before first use)."""
    dev = _need_cuda(workspace)
    _check(lib.aaren_workspace_clear(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(dev)))


@_on_tensor_device
def aaren_scan(q, k, v, scale=None, out_dtype=None, out=None, workspace=None, lse=None,
               return_lse=False):
    """Many-to-many output. q [H,d], k,v [B,H,N,d] -> o [B,H,N,d] (and, with
    return_lse or a given lse tensor, the log-normaliser [B,H,N] float32,
    through aaren_scan_lse)."""
    dev = _need_cuda(q, k, v, out, workspace, lse)
    B, H, N, d = k.shape
    if q.shape != (H, d) or v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("expected q [H,d] and k, v [B,H,N,d] of one dtype")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
    elif out.shape != k.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,H,N,d] of out_dtype")
    if return_lse and lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    need = aaren_scan_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("scan", need, dev, True)
    sc = default_scale(d) if scale is None else float(scale)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if lse is None:
        _check(lib.aaren_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, sc,
                              _dtype_code(k.dtype), _dtype_code(out_dtype), _ptr(ws), wsb,
                              _stream(dev)))
    else:
        if lse.shape != (B, H, N) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B,H,N]")
        _check(lib.aaren_scan_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                  sc, _dtype_code(k.dtype), _dtype_code(out_dtype), _ptr(ws),
                                  wsb, _stream(dev)))
    _debug_check(ws, "aaren_scan")
    return (out, lse) if (return_lse or lse is not None) else out


@_on_tensor_device
def aaren_scan_noalloc(q, k, v, scale=None, out_dtype=None, out=None):
    """aaren_scan with the library's static per-GPU workspace (no workspace
    argument, nothing allocated by the library; `out` may be given so that
    nothing is allocated here either). Shapes needing more than 64 MiB of
    scan workspace are rejected."""
    dev = _need_cuda(q, k, v, out)
    B, H, N, d = k.shape
    if q.shape != (H, d) or v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("expected q [H,d] and k, v [B,H,N,d] of one dtype")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
    elif out.shape != k.shape or out.dtype != out_dtype:
        raise ValueError("out must be [B,H,N,d] of out_dtype")
    _check(lib.aaren_scan_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d,
                                  default_scale(d) if scale is None else float(scale),
                                  _dtype_code(k.dtype), _dtype_code(out_dtype), _stream(dev)))
    return out


def aaren_scan_lse(q, k, v, scale=None, out_dtype=None, out=None, workspace=None, lse=None):
    """aaren_scan with the log-normaliser: returns (o, lse [B,H,N] float32)."""
    return aaren_scan(q, k, v, scale, out_dtype, out, workspace, lse, return_lse=True)


@_on_tensor_device
def aaren_scan_segmented(q, k, v, offsets, scale=None, out_dtype=None, out=None, workspace=None,
                         lse=None, return_lse=False):
    """Each packed sequence scanned on its own. q [H,d], k,v [T,H,d],
    offsets int64 [num_seqs+1] on the device -> o [T,H,d] (and, with
    return_lse or a given lse tensor, the log-normaliser [T,H] float32,
    through aaren_scan_segmented_lse)."""
    dev = _need_cuda(q, k, v, offsets, out, workspace, lse)
    T, H, d = k.shape
    if q.shape != (H, d) or v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("expected q [H,d] and k, v [T,H,d] of one dtype")
    if offsets.dtype != torch.int64 or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be a 1-D int64 tensor of num_seqs+1 entries")
    S = offsets.numel() - 1
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(T, H, d, dtype=out_dtype, device=dev)
    elif out.shape != k.shape or out.dtype != out_dtype:
        raise ValueError("out must be [T,H,d] of out_dtype")
    if return_lse and lse is None:
        lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    need = aaren_scan_segmented_workspace_size(S, T, H, d)
    ws = workspace if workspace is not None else _workspace("scan", need, dev, True)
    sc = default_scale(d) if scale is None else float(scale)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    if lse is None:
        _check(lib.aaren_scan_segmented(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(offsets), S,
                                        T, H, d, sc, _dtype_code(k.dtype),
                                        _dtype_code(out_dtype), _ptr(ws), wsb, _stream(dev)))
    else:
        if lse.shape != (T, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [T,H]")
        _check(lib.aaren_scan_segmented_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                            _ptr(offsets), S, T, H, d, sc, _dtype_code(k.dtype),
                                            _dtype_code(out_dtype), _ptr(ws), wsb,
                                            _stream(dev)))
    _debug_check(ws, "aaren_scan_segmented")
    return (out, lse) if (return_lse or lse is not None) else out


def aaren_scan_segmented_lse(q, k, v, offsets, scale=None, out_dtype=None, out=None,
                             workspace=None, lse=None):
    """aaren_scan_segmented with the log-normaliser: returns (o, lse [T,H])."""
    return aaren_scan_segmented(q, k, v, offsets, scale, out_dtype, out, workspace, lse,
                                return_lse=True)


def aaren_scan_backward_workspace_size(B, H, N, d) -> int:
    return int(lib.aaren_scan_backward_workspace_size(B, H, N, d))


def _backward_dtypes(q, k, v, o, dout, lse):
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or \
            k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v and dout must share one dtype, float32 or bfloat16")
    if o.dtype != torch.float32 or lse.dtype != torch.float32:
        raise TypeError("o and lse must be float32 (the forward's float32 outputs)")


@_on_tensor_device
def aaren_scan_backward(q, k, v, o, dout, lse, scale=None, dq=None, dk=None, dv=None,
                        workspace=None):
    """Gradients of the dense many-to-many scan: (dq [H,d], dk, dv [B,H,N,d]),
    float32, from the forward's o and lse and the output gradient dout. q, k,
    v and dout share one dtype (float32 or bfloat16); o and lse are float32."""
    dev = _need_cuda(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    B, H, N, d = k.shape
    _backward_dtypes(q, k, v, o, dout, lse)
    if q.shape != (H, d) or not (v.shape == o.shape == dout.shape == k.shape) or \
            lse.shape != (B, H, N):
        raise ValueError("expected q [H,d], k, v, o, dout [B,H,N,d] and lse [B,H,N]")
    dq = torch.empty(H, d, dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev) if dv is None else dv
    need = aaren_scan_backward_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("scan", need, dev, True)
    _check(lib.aaren_scan_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                   default_scale(d) if scale is None else float(scale),
                                   _dtype_code(k.dtype), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(dev)))
    _debug_check(ws, "aaren_scan_backward")
    return dq, dk, dv


@_on_tensor_device
def aaren_state_init(m, u, w):
    """Write the empty state into m, u [S,H] and w [S,H,d] (float32)."""
    dev = _need_cuda(m, u, w)
    S, H, d = w.shape
    if m.shape != (S, H) or u.shape != (S, H) or not all(
            t.dtype == torch.float32 for t in (m, u, w)):
        raise ValueError("state must be float32 m, u [S,H] and w [S,H,d]")
    _check(lib.aaren_state_init(_ptr(m), _ptr(u), _ptr(w), S, H, d, _stream(dev)))
    return m, u, w


def new_state(S, H, d, device="cuda"):
    """Allocate (m, u, w) and write the empty state into it."""
    m = torch.empty(S, H, dtype=torch.float32, device=device)
    u = torch.empty(S, H, dtype=torch.float32, device=device)
    w = torch.empty(S, H, d, dtype=torch.float32, device=device)
    return aaren_state_init(m, u, w)


@_on_tensor_device
def aaren_step(q, k_t, v_t, m, u, w, scale=None, out_dtype=None, o_t=None, emit=True):
    """Absorb one pair per (stream, head) into (m, u, w) in place; returns o_t
    [S,H,d] (or None with emit=False)."""
    dev = _need_cuda(q, k_t, v_t, m, u, w, o_t)
    S, H, d = k_t.shape
    if q.shape != (H, d) or v_t.shape != k_t.shape or w.shape != k_t.shape:
        raise ValueError("expected q [H,d], k_t, v_t, w [S,H,d], m, u [S,H]")
    if m.shape != (S, H) or u.shape != (S, H) or not all(
            t.dtype == torch.float32 for t in (m, u, w)):
        raise ValueError("state must be float32 m, u [S,H] and w [S,H,d]")
    out_dtype = out_dtype or torch.float32
    if emit and o_t is None:
        o_t = torch.empty(S, H, d, dtype=out_dtype, device=dev)
    _check(lib.aaren_step(_ptr(q), _ptr(k_t), _ptr(v_t), _ptr(m), _ptr(u), _ptr(w),
                          _ptr(o_t if emit else None), S, H, d,
                          default_scale(d) if scale is None else float(scale),
                          _dtype_code(k_t.dtype), _dtype_code(out_dtype), _stream(dev)))
    return o_t if emit else None


@_on_tensor_device
def aaren_append(q, k, v, m, u, w, scale=None, out_dtype=None, o=None, emit=True):
    """Append T pairs per (stream, head) to (m, u, w) in place: k, v [T,S,H,d]
    time-major; returns o [T,S,H,d] (or None with emit=False)."""
    dev = _need_cuda(q, k, v, m, u, w, o)
    T, S, H, d = k.shape
    if q.shape != (H, d) or v.shape != k.shape or w.shape != (S, H, d):
        raise ValueError("expected q [H,d], k, v [T,S,H,d], w [S,H,d], m, u [S,H]")
    if q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("q, k and v must share one dtype")
    if m.shape != (S, H) or u.shape != (S, H) or not all(
            t.dtype == torch.float32 for t in (m, u, w)):
        raise ValueError("state must be float32 m, u [S,H] and w [S,H,d]")
    out_dtype = out_dtype or torch.float32
    if emit and o is None:
        o = torch.empty(T, S, H, d, dtype=out_dtype, device=dev)
    _check(lib.aaren_append(_ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(u), _ptr(w),
                            _ptr(o if emit else None), S, T, H, d,
                            default_scale(d) if scale is None else float(scale),
                            _dtype_code(k.dtype), _dtype_code(out_dtype), _stream(dev)))
    return o if emit else None


@_on_tensor_device
def aaren_scan_strided(q, k, v, scale=None, out_dtype=None, out=None, workspace=None, lse=None,
                       return_lse=False):
    """aaren_scan over k, v given as [B,H,N,d] views with any strides whose
    last dimension is contiguous (e.g. token-major [B,N,H,d] memory permuted
    to [B,H,N,d]); out has k's layout unless given."""
    dev = _need_cuda(q, k, v, out, workspace, lse, strided=(k, v, out))
    B, H, N, d = k.shape
    if v.shape != k.shape or v.stride() != k.stride() or q.shape != (H, d):
        raise ValueError("expected q [H,d] and k, v [B,H,N,d] views with equal strides")
    if k.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty_like(k, dtype=out_dtype)
    if out.shape != k.shape or out.stride(3) != 1:
        raise ValueError("out must be a [B,H,N,d] view with a contiguous last dimension")
    if lse is None and return_lse:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    kvs = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    os_ = (ctypes.c_int64 * 3)(out.stride(0), out.stride(1), out.stride(2))
    need = aaren_scan_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("scan", need, dev, True)
    _check(lib.aaren_scan_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                  kvs, os_, default_scale(d) if scale is None else float(scale),
                                  _dtype_code(k.dtype), _dtype_code(out.dtype), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(dev)))
    _debug_check(ws, "aaren_scan_strided")
    return (out, lse) if (return_lse or lse is not None) else out


def aaren_layer_workspace_size(B, N, Dm, H, d) -> int:
    return int(lib.aaren_layer_workspace_size(B, N, Dm, H, d))


@_on_tensor_device
def aaren_layer_forward(x, w_kv, q, scale=None, out_dtype=None, out=None, workspace=None):
    """One Aaren layer: x [B,N,Dm] bf16, w_kv [Dm, 2*H*d] bf16 (W_K | W_V),
    q [H,d] float32 -> o [B,N,H,d] (bf16 by default, so that layers stack)."""
    dev = _need_cuda(x, w_kv, q, out, workspace)
    B, N, Dm = x.shape
    H, d = q.shape
    if w_kv.shape != (Dm, 2 * H * d) or x.dtype != torch.bfloat16 or w_kv.dtype != torch.bfloat16:
        raise ValueError("expected bf16 x [B,N,Dm] and w_kv [Dm, 2*H*d]")
    if q.dtype != torch.float32:
        raise ValueError("q must be float32 [H,d]")
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty(B, N, H, d, dtype=out_dtype, device=dev)
    aaren_init(dev)  # once per device: the projection's rocBLAS handle
    need = aaren_layer_workspace_size(B, N, Dm, H, d)
    ws = workspace if workspace is not None else _workspace("layer", need, dev, True)
    _check(lib.aaren_layer_forward(_ptr(x), _ptr(w_kv), _ptr(q), _ptr(out), B, N, Dm, H, d,
                                   default_scale(d) if scale is None else float(scale),
                                   _dtype_code(out.dtype), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(dev)))
    return out


def aaren_scan_segmented_backward_workspace_size(num_seqs, total_tokens, H, d) -> int:
    return int(lib.aaren_scan_segmented_backward_workspace_size(num_seqs, total_tokens, H, d))


@_on_tensor_device
def aaren_scan_segmented_backward(q, k, v, o, dout, lse, offsets, scale=None, dq=None, dk=None,
                                  dv=None, workspace=None):
    """Gradients of the packed scan: q [H,d]; k, v, dout [T,H,d] (float32 or
    bfloat16, one dtype); o [T,H,d] and lse [T,H] float32 from
    aaren_scan_segmented; offsets int64 [S+1] -> (dq, dk, dv) float32."""
    dev = _need_cuda(q, k, v, o, dout, lse, offsets, dq, dk, dv, workspace)
    T, H, d = k.shape
    _backward_dtypes(q, k, v, o, dout, lse)
    for t in (v, o, dout):
        if t.shape != k.shape:
            raise ValueError("k, v, o, dout must share one [T,H,d] shape")
    if lse.shape != (T, H) or offsets.dtype != torch.int64 or offsets.dim() != 1:
        raise ValueError("expected lse [T,H] and int64 offsets [S+1]")
    S = offsets.numel() - 1
    dq = dq if dq is not None else torch.empty(H, d, device=dev)
    dk = dk if dk is not None else torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = dv if dv is not None else torch.empty(v.shape, dtype=torch.float32, device=dev)
    need = aaren_scan_segmented_backward_workspace_size(S, T, H, d)
    ws = workspace if workspace is not None else _workspace("segbwd", need, dev, True)
    _check(lib.aaren_scan_segmented_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(offsets), _ptr(dq), _ptr(dk),
        _ptr(dv), S, T, H, d, default_scale(d) if scale is None else float(scale),
        _dtype_code(k.dtype), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(dev)))
    _debug_check(ws, "aaren_scan_segmented_backward")
    return dq, dk, dv


def aaren_mean_query_attention_workspace_size(B, H, N, d) -> int:
    return int(lib.aaren_mean_query_attention_workspace_size(B, H, N, d))


@_on_tensor_device
def aaren_mean_query_attention(hq, k, v, scale=None, out_dtype=None, out=None, g_out=None,
                               return_query=False, workspace=None):
    """Attention of each (b,h)'s mean query over all its pairs: hq, k, v
    [B,H,N,d] -> o [B,H,d] (and the mean queries g [B,H,d] float32)."""
    dev = _need_cuda(hq, k, v, out, g_out, workspace)
    B, H, N, d = k.shape
    if hq.shape != k.shape or v.shape != k.shape or not (hq.dtype == k.dtype == v.dtype):
        raise ValueError("expected hq, k, v [B,H,N,d] of one dtype")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(B, H, d, dtype=out_dtype, device=dev)
    if g_out is None and return_query:
        g_out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    need = aaren_mean_query_attention_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("meanq", need, dev, False)
    _check(lib.aaren_mean_query_attention(_ptr(hq), _ptr(k), _ptr(v), _ptr(out), _ptr(g_out), B, H,
                                          N, d, default_scale(d) if scale is None else float(scale),
                                          _dtype_code(k.dtype), _dtype_code(out.dtype), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(),
                                          _stream(dev)))
    return (out, g_out) if (return_query or g_out is not None) else out


def aaren_self_attention_workspace_size(B, H, N, d) -> int:
    return int(lib.aaren_self_attention_workspace_size(B, H, N, d))


@_on_tensor_device
def aaren_self_attention(q, k, v, scale=None, causal=True, out_dtype=None, out=None, lse=None,
                         return_lse=False, workspace=None):
    """Self-attention, one query per token: q, k, v [B,H,N,d] bfloat16 -> o
    [B,H,N,d] (and lse [B,H,N] float32 with return_lse or a given lse)."""
    dev = _need_cuda(q, k, v, out, lse, workspace)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("expected q, k, v [B,H,N,d] of one dtype")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(B, H, N, d, dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    need = aaren_self_attention_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("attn", need, dev, False)
    _check(lib.aaren_self_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                    default_scale(d) if scale is None else float(scale),
                                    int(bool(causal)), _dtype_code(q.dtype), _dtype_code(out.dtype),
                                    _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


@_on_tensor_device
def aaren_reduce(q, k, v, scale=None, out_dtype=None, stats=False, out=None, workspace=None):
    """Many-to-one output. q [H,d], k,v [B,H,N,d] -> o [B,H,d] (and, with
    stats, the final state's m and u [B,H] float32)."""
    dev = _need_cuda(q, k, v, out, workspace)
    B, H, N, d = k.shape
    if q.shape != (H, d) or v.shape != k.shape or q.dtype != k.dtype or v.dtype != k.dtype:
        raise ValueError("expected q [H,d] and k, v [B,H,N,d] of one dtype")
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(B, H, d, dtype=out_dtype, device=dev)
    m = torch.empty(B, H, dtype=torch.float32, device=dev) if stats else None
    u = torch.empty(B, H, dtype=torch.float32, device=dev) if stats else None
    need = aaren_reduce_workspace_size(B, H, N, d)
    ws = workspace if workspace is not None else _workspace("reduce", need, dev, False)
    _check(lib.aaren_reduce(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(u), B, H, N, d,
                            default_scale(d) if scale is None else float(scale),
                            _dtype_code(k.dtype), _dtype_code(out_dtype), _ptr(ws),
                            0 if ws is None else ws.numel() * ws.element_size(), _stream(dev)))
    return (out, m, u) if stats else out
