"""The workspace's error word through the C ABI (aaren_workspace_status).

The condition is forced from the host: a ticket counter of a fresh
workspace is set out of range before the first call, so the workgroup that
draws it refuses at once and notes bit 0; every other workgroup draws a
valid position and the kernel ends normally (nothing waits on the refused
tile: it would have been its stream's last). The workspace comes straight
from hipMalloc, at an address no earlier call has used, so the library
takes it as zero-filled and clears nothing before the call."""
import ctypes

import pytest
import torch

import exact_softmax_attention_02_amd as aaren
import oracle
from _gpu import announce, dev, host32

pytestmark = pytest.mark.gpu

HEADER = 256          # bytes before the ticket counters
ERROR_WORD = slice(12, 16)

_hip = ctypes.CDLL("libamdhip64.so")
_hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
_hip.hipFree.argtypes = [ctypes.c_void_p]
_hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
H2D, D2H = 1, 2


def _inputs(B, H, N, d, seed):
    g = torch.Generator(device=dev()).manual_seed(seed)
    return (torch.randn(*s, generator=g, device=dev()) for s in ((H, d), (B, H, N, d), (B, H, N, d)))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_out_of_range_ticket_is_reported_and_reset():
    announce("workspace status: a ticket counter set out of range")
    B, H, N, d = 1, 2, 1024, 64        # 5 tiles per stream (3 full, 2 half), no padding
    q, k, v = _inputs(B, H, N, d, 62)
    o = torch.empty_like(k)
    need = aaren.aaren_scan_workspace_size(B, H, N, d)
    ws = ctypes.c_void_p()
    torch.cuda.synchronize()
    assert _hip.hipMalloc(ctypes.byref(ws), need) == 0
    try:
        host = (ctypes.c_uint8 * need)()
        ctypes.c_uint32.from_buffer(host, HEADER).value = 1000   # stream 0's counter
        assert _hip.hipMemcpy(ws, host, need, H2D) == 0
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = aaren.lib.aaren_scan(_p(q), _p(k), _p(v), _p(o), B, H, N, d,
                                  aaren.default_scale(d), aaren.AAREN_F32, aaren.AAREN_F32,
                                  ws, need, stream)
        assert st == aaren.AAREN_OK
        flags = torch.full((2,), -1, dtype=torch.int32, device=dev())
        assert aaren.lib.aaren_workspace_status(ws, need, _p(flags), 1, stream) == 0
        assert aaren.lib.aaren_workspace_status(ws, need, ctypes.c_void_p(flags.data_ptr() + 4),
                                                0, stream) == 0
        torch.cuda.synchronize()
        first, after_reset = (int(x) for x in flags.cpu())
        assert first & 1, first           # the refused draw
        assert after_reset == 0           # reset=1 cleared the word after copying it

        # zero-filled again through the ABI, the same workspace gives the oracle's result
        assert aaren.lib.aaren_workspace_clear(ws, need, stream) == 0
        o.zero_()
        assert aaren.lib.aaren_scan(_p(q), _p(k), _p(v), _p(o), B, H, N, d,
                                    aaren.default_scale(d), aaren.AAREN_F32, aaren.AAREN_F32,
                                    ws, need, stream) == 0
        assert aaren.lib.aaren_workspace_status(ws, need, _p(flags), 0, stream) == 0
        torch.cuda.synchronize()
        assert int(flags[0]) == 0
        ref = oracle.scan(host32(q), host32(k), host32(v), aaren.default_scale(d))
        assert oracle.max_scaled_err(host32(o), ref) <= 1e-5
    finally:
        torch.cuda.synchronize()
        _hip.hipFree(ws)


def test_debug_mode_raises_on_a_flagged_workspace(monkeypatch):
    """With AAREN_DEBUG the binding reads the word after every scan: a
    workspace whose word is set (here written by the test) makes the call
    raise; a clean one does not."""
    announce("workspace status: debug mode of the binding")
    q, k, v = _inputs(2, 3, 1000, 64, 61)
    ws = torch.zeros(aaren.aaren_scan_workspace_size(2, 3, 1000, 64), dtype=torch.uint8,
                     device=dev())
    monkeypatch.setattr(aaren, "_DEBUG", True)
    for _ in range(3):
        aaren.aaren_scan(q, k, v, workspace=ws)          # checked, clean
    assert aaren.aaren_workspace_status(ws) == 0
    ws[ERROR_WORD].view(torch.int32).fill_(4)
    with pytest.raises(aaren.AarenError, match="error flags 0x4"):
        aaren.aaren_scan(q, k, v, workspace=ws)
    assert aaren.aaren_workspace_status(ws, reset=True) == 4
    assert aaren.aaren_workspace_status(ws) == 0
    aaren.aaren_scan(q, k, v, workspace=ws)
