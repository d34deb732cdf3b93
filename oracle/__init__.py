"""CPU oracle for single-query softmax attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. It never touches the GPU library and shares no code with it.

Two independent evaluations of the same definition live here:

* ``aaren_oracle.c`` -- the constant-memory recurrence of the "Self-attention
  Does Not Need O(n^2) Memory" review (section 2 Algorithm), stabilised by a
  running maximum, in float64 with OpenMP over independent units. It is fast
  enough for every workload at full size.
* ``brute.py`` -- the definition written out (softmax of all prefix scores,
  then the weighted sum), O(N^2 d), plus the combine operator used to check
  that any bracketing of the scan gives the same result.

The functions below take numpy arrays (float32 inputs; bfloat16 inputs must be
widened to float32 by the caller, which is exact) and return float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aaren_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP). Returns its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the argument and result types of a loaded oracle library."""
    f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
    f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
    i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
    opt64 = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_scan.argtypes = [f32p, f32p, f32p, i64, i64, i64, i64, ctypes.c_double,
                                f64p, opt64, opt64]
    lib.oracle_scan_f64.argtypes = [f64p, f64p, f64p, i64, i64, i64, i64, ctypes.c_double, f64p]
    lib.oracle_scan_segmented.argtypes = [f32p, f32p, f32p, i64p, i64, i64, i64, i64,
                                          ctypes.c_double, f64p, opt64, opt64]
    lib.oracle_step.argtypes = [f32p, f32p, f32p, f64p, f64p, f64p, opt64,
                                i64, i64, i64, ctypes.c_double]
    lib.oracle_reduce.argtypes = [f32p, f32p, f32p, i64, i64, i64, i64, ctypes.c_double,
                                  f64p, opt64, opt64]
    lib.oracle_scan_backward.argtypes = [f32p, f32p, f32p, f32p, i64, i64, i64, i64,
                                         ctypes.c_double, f64p, f64p, f64p]
    lib.oracle_self_attention.argtypes = [f32p, f32p, f32p, i64, i64, i64, i64, ctypes.c_double,
                                          ctypes.c_int, i64, i64, f64p, opt64]
    for fn in (lib.oracle_scan, lib.oracle_scan_f64, lib.oracle_scan_segmented, lib.oracle_step,
               lib.oracle_reduce, lib.oracle_scan_backward):
        fn.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _configure(ctypes.CDLL(build()))
    return _lib


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle inputs are float32 (got {a.dtype}); widen bfloat16 first")
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the loops over independent units (timing only)."""
    _load().oracle_set_threads(int(n))


def scan(q, k, v, scale, stats: bool = False):
    """Many-to-many output. q [H,d], k,v [B,H,N,d] float32 -> o [B,H,N,d] float64
    (and, with stats, the running max m and L = m + ln u, both [B,H,N])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = k.shape
    assert q.shape == (H, d) and v.shape == k.shape
    o = np.empty((B, H, N, d), np.float64)
    m = np.empty((B, H, N), np.float64) if stats else None
    lse = np.empty((B, H, N), np.float64) if stats else None
    rc = _load().oracle_scan(q, k, v, B, H, N, d, float(scale), o, _ptr(m), _ptr(lse))
    if rc:
        raise ValueError("oracle_scan rejected its arguments")
    return (o, m, lse) if stats else o


def scan_f64(q, k, v, scale):
    """The many-to-many output for float64 inputs (keys and values that are
    not float32 values, such as the layer's projections): q [H,d], k, v
    [B,H,N,d] -> o [B,H,N,d] float64, the same recurrence as scan()."""
    q, k, v = (np.ascontiguousarray(np.asarray(a, np.float64)) for a in (q, k, v))
    B, H, N, d = k.shape
    assert q.shape == (H, d) and v.shape == k.shape
    o = np.empty((B, H, N, d), np.float64)
    if _load().oracle_scan_f64(q, k, v, B, H, N, d, float(scale), o):
        raise ValueError("oracle_scan_f64 rejected its arguments")
    return o


def scan_segmented(q, k, v, offsets, scale, stats: bool = False):
    """Each packed sequence scanned on its own. q [H,d], k,v [T,H,d] float32,
    offsets int64 [S+1] -> o [T,H,d] float64 (and m, L [T,H] with stats)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    offsets = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    T, H, d = k.shape
    S = offsets.size - 1
    o = np.empty((T, H, d), np.float64)
    m = np.empty((T, H), np.float64) if stats else None
    lse = np.empty((T, H), np.float64) if stats else None
    rc = _load().oracle_scan_segmented(q, k, v, offsets, S, T, H, d, float(scale), o,
                                       _ptr(m), _ptr(lse))
    if rc:
        raise ValueError("oracle_scan_segmented rejected its arguments")
    return (o, m, lse) if stats else o


def state_init(S, H, d):
    """A fresh (empty) state: m = -inf, u = 0, w = 0."""
    return (np.full((S, H), -np.inf), np.zeros((S, H)), np.zeros((S, H, d)))


def step(q, k_t, v_t, state, scale):
    """Absorb one pair per (stream, head) into state = (m, u, w) (float64,
    updated in place) and return o_t [S,H,d] float64."""
    q, k_t, v_t = _f32(q), _f32(k_t), _f32(v_t)
    S, H, d = k_t.shape
    m, u, w = state
    for a in (m, u, w):
        assert a.dtype == np.float64 and a.flags.c_contiguous
    o = np.empty((S, H, d), np.float64)
    rc = _load().oracle_step(q, k_t, v_t, m, u, w, _ptr(o), S, H, d, float(scale))
    if rc:
        raise ValueError("oracle_step rejected its arguments")
    return o


def scan_segmented_backward(q, k, v, dout, offsets, scale):
    """Gradients of the packed many-to-many output: q [H,d]; k, v, dout [T,H,d];
    offsets [S+1]. Each sequence is scanned on its own, so its gradients are
    the dense gradients of that sequence (scan_backward), and dq adds every
    sequence's dq. Returns dq [H,d], dk, dv [T,H,d] float64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    offsets = np.asarray(offsets, np.int64)
    T, H, d = k.shape
    dq = np.zeros((H, d), np.float64)
    dk = np.zeros((T, H, d), np.float64)
    dv = np.zeros((T, H, d), np.float64)
    for s in range(offsets.size - 1):
        a, b = int(offsets[s]), int(offsets[s + 1])
        if a == b:
            continue
        per = [np.ascontiguousarray(x[a:b].transpose(1, 0, 2)[None]) for x in (k, v, dout)]
        rq, rk, rv = scan_backward(q, per[0], per[1], per[2], scale)
        dq += rq
        dk[a:b] = rk[0].transpose(1, 0, 2)
        dv[a:b] = rv[0].transpose(1, 0, 2)
    return dq, dk, dv


def append(q, k, v, state, scale):
    """Append T tokens to every (stream, head) state: k, v [T,S,H,d]
    (time-major, k[t] is one step's keys), state = (m, u, w) float64 updated
    in place; returns o [T,S,H,d] float64, o[t] the output after token t.

    By definition T successive single-pair updates: the RNN view of the
    "Attention as an RNN" review (abstract item (ii), proposed method) absorbs
    new tokens one at a time into the constant-size state."""
    k, v = _f32(k), _f32(v)
    out = np.empty(k.shape, np.float64)
    for t in range(k.shape[0]):
        out[t] = step(q, k[t], v[t], state, scale)
    return out


def reduce(q, k, v, scale, stats: bool = False):
    """Many-to-one output. q [H,d], k,v [B,H,N,d] -> o [B,H,d] float64
    (and m, L [B,H] with stats)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = k.shape
    o = np.empty((B, H, d), np.float64)
    m = np.empty((B, H), np.float64) if stats else None
    lse = np.empty((B, H), np.float64) if stats else None
    rc = _load().oracle_reduce(q, k, v, B, H, N, d, float(scale), o, _ptr(m), _ptr(lse))
    if rc:
        raise ValueError("oracle_reduce rejected its arguments")
    return (o, m, lse) if stats else o


def scan_backward(q, k, v, dout, scale):
    """Gradients of the many-to-many output given dout: q [H,d], k, v, dout
    [B,H,N,d] float32 -> (dq [H,d], dk, dv [B,H,N,d]) float64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, N, d = k.shape
    assert q.shape == (H, d) and v.shape == k.shape and dout.shape == k.shape
    dq = np.empty((H, d), np.float64)
    dk = np.empty((B, H, N, d), np.float64)
    dv = np.empty((B, H, N, d), np.float64)
    rc = _load().oracle_scan_backward(q, k, v, dout, B, H, N, d, float(scale), dq, dk, dv)
    if rc:
        raise ValueError("oracle_scan_backward rejected its arguments")
    return dq, dk, dv


def self_attention(q, k, v, scale, causal: bool = True, rows=None, stats: bool = False):
    """Self-attention with one query per token: q, k, v [B,H,N,d] -> o
    [B,H,R,d] float64 for query rows rows = (begin, end) (all rows if None),
    each the single-query recurrence over pairs 0..i (causal) or all pairs;
    with stats also L [B,H,R] (log-normaliser, natural units)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = k.shape
    a, b = (0, N) if rows is None else (int(rows[0]), int(rows[1]))
    o = np.empty((B, H, b - a, d), np.float64)
    lse = np.empty((B, H, b - a), np.float64) if stats else None
    rc = _load().oracle_self_attention(q, k, v, B, H, N, d, float(scale), int(bool(causal)), a, b,
                                       o, _ptr(lse))
    if rc:
        raise ValueError("oracle_self_attention rejected its arguments")
    return (o, lse) if stats else o


def mean_query_attention(hq, k, v, scale, stats: bool = False):
    """Global-aggregation attention of the pooling network on the
    efficient-transformer page (PoNet, "Global aggregation" and its two
    equations): per (b,h) the query g is the mean of hq over the N tokens,
    and o is the attention of g over all N pairs: the softmax of the scores
    scale <g, k_n> weighting the values. Everything in float64 (g is not
    rounded). hq, k, v [B,H,N,d] -> o [B,H,d] (and g [B,H,d] float64)."""
    hq, k, v = _f32(hq), _f32(k), _f32(v)
    B, H, N, d = k.shape
    g = hq.astype(np.float64).mean(axis=2)
    o = np.empty((B, H, d), np.float64)
    for b in range(B):
        for h in range(H):
            s = float(scale) * (k[b, h].astype(np.float64) @ g[b, h])
            p = np.exp(s - s.max())
            o[b, h] = (p @ v[b, h].astype(np.float64)) / p.sum()
    return (o, g) if stats else o


def bf16_round(a):
    """Round float64 values to the nearest bfloat16 value (8 significant
    bits), ties to even; returned as float64. Normal range only."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                       # a = m 2^e, 1/2 <= |m| < 1
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def layer_forward(x, w_kv, q, scale, out_bf16: bool = True):
    """One Aaren layer: x [B,N,Dm], w_kv [Dm, 2*H*d] (W_K | W_V), q [H,d]
    -> o [B,N,H,d] float64. [K | V] = x w_kv in float64, then the
    many-to-many scan of q_h over each (b, h) in float64 ("Attention as an
    RNN" review, proposed method: a learned query, the prefix-scan output);
    with out_bf16 the output is rounded to bfloat16, the precision a stacked
    layer receives."""
    x, w_kv, q = (np.asarray(t, np.float64) for t in (x, w_kv, q))
    B, N, Dm = x.shape
    H, d = q.shape
    kv = (x.reshape(B * N, Dm) @ w_kv).reshape(B, N, 2, H, d)
    k = np.ascontiguousarray(kv[:, :, 0].transpose(0, 2, 1, 3))   # [B,H,N,d]
    v = np.ascontiguousarray(kv[:, :, 1].transpose(0, 2, 1, 3))
    o = scan_f64(q, k, v, scale).transpose(0, 2, 1, 3)  # [B,N,H,d]
    return bf16_round(o) if out_bf16 else np.ascontiguousarray(o)


def max_scaled_err(got, ref) -> float:
    """max over elements of |got - ref| / (1 + |ref|): the error measure the
    tolerances are stated in. NaN where either side is NaN counts as failure
    unless both are NaN."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if got.size == 0:
        return 0.0
    both_nan = np.isnan(got) & np.isnan(ref)
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    err = np.where(both_nan, 0.0, err)
    if np.isnan(err).any():
        return float("inf")
    return float(err.max())
