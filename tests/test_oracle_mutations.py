"""Plant a plausible mistake in a copy of the oracle and require the pins to
catch it (no GPU). Each mutant is compiled into a temporary directory; the
real oracle is never modified."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import _pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "aaren_oracle.c")

# (name, function the edit is confined to or None for the whole file, old, new)
MUTATIONS = [
    ("rescale exponent sign flipped", None, "exp(*m - s)", "exp(s - *m)"),
    ("normaliser not rescaled", None, "*u = *u * shrink + 1.0;", "*u = *u + 1.0;"),
    ("value sum not rescaled", None, "w[j] = w[j] * shrink + (double)v[j];",
     "w[j] = w[j] + (double)v[j];"),
    ("no max subtraction", None, "double p = exp(s - *m);", "double p = exp(s);"),
    ("running max starts at 0, not -inf", "oracle_scan", "double m = -INFINITY, u = 0.0;",
     "double m = 0.0, u = 0.0;"),
    ("running max never raised", None, "*m = s;", ";"),
    ("new-maximum term weighted by e^s", None, "*u = *u * shrink + 1.0;",
     "*u = *u * shrink + exp(s);"),
    ("key index wrong", None, "(double)q[j] * (double)k[j]", "(double)q[j] * (double)k[0]"),
    ("scale dropped", None, "return scale * acc;", "return acc;"),
    ("scale applied twice", None, "return scale * acc;", "return scale * scale * acc;"),
    ("no final division", None, "o[j] = w[j] / u;", "o[j] = w[j];"),
    ("log-normaliser without max", None, "*lse_out = m + log(u);", "*lse_out = log(u);"),
    ("exclusive instead of inclusive output", "oracle_scan",
     "absorb(&m, &u, w, d, score(qh, k + row * d, d, scale), v + row * d);\n"
     "                emit(m, u, w, d, o + row * d, m_out ? m_out + row : NULL,\n"
     "                     lse_out ? lse_out + row : NULL);",
     "if (i == 0) { for (int64_t j = 0; j < d; ++j) o[row * d + j] = 0.0; }\n"
     "                else emit(m, u, w, d, o + row * d, m_out ? m_out + row : NULL,\n"
     "                     lse_out ? lse_out + row : NULL);\n"
     "                absorb(&m, &u, w, d, score(qh, k + row * d, d, scale), v + row * d);"),
    ("float64 scan: rescale exponent sign flipped", "oracle_scan_f64", "exp(m - sc)",
     "exp(sc - m)"),
    ("float64 scan: value sum not rescaled", "oracle_scan_f64",
     "w[j] = w[j] * shrink + vr[j];", "w[j] = w[j] + vr[j];"),
    ("float64 scan: query of head 0 for all heads", "oracle_scan_f64",
     "const double *qh = q + (unit % H) * d;", "const double *qh = q;"),
    ("segmented: query of head 0 for all heads", "oracle_scan_segmented",
     "score(q + h * d, k + row * d", "score(q, k + row * d"),
    ("segmented: head stride dropped", "oracle_scan_segmented",
     "int64_t row = t * H + h;", "int64_t row = t * H + (h > 0 ? h - 1 : 0);"),
    ("segmented: state not restarted per sequence", "oracle_scan_segmented",
     "for (int64_t t = offsets[seq]; t < offsets[seq + 1]; ++t) {",
     "for (int64_t t = (seq > 0 ? offsets[seq - 1] : 0); t < offsets[seq + 1]; ++t) {"),
    ("step: key and value swapped", "oracle_step", "score(qh, k_t + unit * d",
     "score(qh, v_t + unit * d"),
    ("step: query of the wrong head", "oracle_step", "const float *qh = q + (unit % H) * d;",
     "const float *qh = q + (unit / H % H) * d;"),
    ("reduce drops the last pair", "oracle_reduce", "for (int64_t i = 0; i < N; ++i)",
     "for (int64_t i = 0; i < N - 1; ++i)"),
    ("reduce reads rows of the wrong unit", "oracle_reduce", "int64_t row = unit * N + i;",
     "int64_t row = (unit % H) * N + i;"),
    ("backward: suffix weight inverted", "oracle_scan_backward", "exp(L[i] - L[i + 1])",
     "exp(L[i + 1] - L[i])"),
    ("backward: <g, v> in place of <g, o>", "oracle_scan_backward",
     "delta += (double)g[j] * o[i * d + j];", "delta += (double)g[j] * (double)v[row * d + j];"),
    ("backward: dv without the diagonal weight", "oracle_scan_backward",
     "dv[row * d + j] = pii * G[j];", "dv[row * d + j] = G[j];"),
    ("backward: score gradient without the output term", "oracle_scan_backward",
     "ds -= pii * D;", ";"),
    ("backward: dk along k instead of q", "oracle_scan_backward",
     "dk[row * d + j] = scale * ds * (double)qh[j];",
     "dk[row * d + j] = scale * ds * (double)k[row * d + j];"),
    ("backward: dq of the first batch row only", "oracle_scan_backward",
     "for (int64_t b = 0; b < B; ++b)", "for (int64_t b = 0; b < 1; ++b)"),
    ("self-attention: causal rows exclude their own pair", "oracle_self_attention",
     "for (int64_t j = 0; j <= last; ++j)", "for (int64_t j = 0; j < (last > 0 ? last : 1); ++j)"),
    ("self-attention: the first query for every row", "oracle_self_attention",
     "const float *qi = q + (unit * N + i) * d;", "const float *qi = q + (unit * N) * d;"),
    ("self-attention: all pairs but the last", "oracle_self_attention",
     "const int64_t last = causal ? i : N - 1;", "const int64_t last = causal ? i : (N > 1 ? N - 2 : 0);"),
    ("self-attention: keys of the wrong head", "oracle_self_attention",
     "const int64_t row = unit * N + j;", "const int64_t row = (unit / H) * H * N + j;"),
]


def _mutate(src, func, old, new):
    if func is None:
        assert old in src, old
        return src.replace(old, new)
    start = src.index("int " + func + "(")
    nxt = src.find("\nint ", start + 1)
    end = len(src) if nxt < 0 else nxt
    body = src[start:end]
    assert old in body, (func, old)
    return src[:start] + body.replace(old, new) + src[end:]


class _Bound:
    """The oracle module's functions, bound to another build of the library."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(oracle, name)
        if not callable(fn):
            return fn

        def call(*a, **kw):
            saved = oracle._lib
            oracle._lib = self._lib
            try:
                return fn(*a, **kw)
            finally:
                oracle._lib = saved
        return call


@pytest.mark.parametrize("name,func,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, func, old, new):
    src = open(SRC).read()
    mutant = tmp_path / "mutant.c"
    mutant.write_text(_mutate(src, func, old, new))
    lib_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w",
                    "-o", str(lib_path), str(mutant), "-lm"], check=True)
    bound = _Bound(oracle._configure(ctypes.CDLL(str(lib_path))))
    caught = []
    for check in _pins.ALL:
        try:
            check(bound)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"


def _append_dropping_last(q, k, v, state, scale):
    out = np.zeros(np.shape(k), np.float64)
    for t in range(max(np.shape(k)[0] - 1, 0)):
        out[t] = oracle.step(q, k[t], v[t], state, scale)
    return out


def _append_previous_value(q, k, v, state, scale):
    out = np.empty(np.shape(k), np.float64)
    for t in range(np.shape(k)[0]):
        out[t] = oracle.step(q, k[t], v[max(t - 1, 0)], state, scale)
    return out


def _append_on_a_copy(q, k, v, state, scale):
    return oracle.append(q, k, v, tuple(a.copy() for a in state), scale)


class _AppendMutant:
    """The oracle with its append replaced by a mistaken one."""

    def __init__(self, fn):
        self.append = fn

    def __getattr__(self, name):
        return getattr(oracle, name)


@pytest.mark.parametrize("fn", [_append_dropping_last, _append_previous_value, _append_on_a_copy],
                         ids=["append drops the last token", "append pairs k_t with v_(t-1)",
                              "append leaves the caller's state unchanged"])
def test_append_mutant_is_caught(fn):
    with pytest.raises((AssertionError, ValueError)):
        _pins.check_append(_AppendMutant(fn))


def _layer_kv_swapped(x, w_kv, q, scale, out_bf16=True):
    H, d = np.shape(q)
    w = np.asarray(w_kv)
    return oracle.layer_forward(x, np.concatenate([w[:, H * d:], w[:, :H * d]], axis=1), q, scale,
                                out_bf16)


def _layer_heads_interleaved(x, w_kv, q, scale, out_bf16=True):
    # reads columns as [d][2][H] instead of [2][H][d]
    H, d = np.shape(q)
    w = np.asarray(w_kv).reshape(-1, d, 2, H).transpose(0, 2, 3, 1).reshape(-1, 2 * H * d)
    return oracle.layer_forward(x, w, q, scale, out_bf16)


def _layer_round_to_zero(x, w_kv, q, scale, out_bf16=True):
    o = oracle.layer_forward(x, w_kv, q, scale, out_bf16=False)
    if not out_bf16:
        return o
    m, e = np.frexp(o)
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


class _LayerMutant:
    def __init__(self, fn):
        self.layer_forward = fn

    def __getattr__(self, name):
        return getattr(oracle, name)


@pytest.mark.parametrize("fn", [_layer_kv_swapped, _layer_heads_interleaved, _layer_round_to_zero],
                         ids=["layer: W_K and W_V swapped", "layer: head columns interleaved",
                              "layer: output truncated instead of rounded"])
def test_layer_mutant_is_caught(fn):
    with pytest.raises(AssertionError):
        _pins.check_layer(_LayerMutant(fn))


def _mean_query_summed(hq, k, v, scale, stats=False):
    hq = np.asarray(hq, np.float32)
    return oracle.mean_query_attention(hq * np.float32(hq.shape[2]), k, v, scale, stats)


def _mean_query_first_token(hq, k, v, scale, stats=False):
    hq = np.asarray(hq, np.float32)
    return oracle.mean_query_attention(np.repeat(hq[:, :, :1], hq.shape[2], axis=2), k, v, scale,
                                       stats)


class _MeanQueryMutant:
    def __init__(self, fn):
        self.mean_query_attention = fn

    def __getattr__(self, name):
        return getattr(oracle, name)


@pytest.mark.parametrize("fn", [_mean_query_summed, _mean_query_first_token],
                         ids=["mean query: sum without 1/N", "mean query: first token only"])
def test_mean_query_mutant_is_caught(fn):
    with pytest.raises(AssertionError):
        _pins.check_mean_query(_MeanQueryMutant(fn))


def _seg_bwd_unseparated(q, k, v, dout, offsets, scale):
    T = np.shape(k)[0]
    return oracle.scan_segmented_backward(q, k, v, dout, np.array([0, T]), scale)


def _seg_bwd_last_dq(q, k, v, dout, offsets, scale):
    dq, dk, dv = oracle.scan_segmented_backward(q, k, v, dout, offsets, scale)
    return _only_last_dq(q, k, v, dout, np.asarray(offsets), scale), dk, dv


def _only_last_dq(q, k, v, dout, o, scale):
    a, b = int(o[-2]), int(o[-1])
    sub = [np.ascontiguousarray(np.asarray(x)[a:b].transpose(1, 0, 2)[None]) for x in (k, v, dout)]
    return oracle.scan_backward(q, sub[0], sub[1], sub[2], scale)[0]


class _SegBwdMutant:
    def __init__(self, fn):
        self.scan_segmented_backward = fn

    def __getattr__(self, name):
        return getattr(oracle, name)


@pytest.mark.parametrize("fn", [_seg_bwd_unseparated, _seg_bwd_last_dq],
                         ids=["packed backward: sequences not separated",
                              "packed backward: dq of the last sequence only"])
def test_segmented_backward_mutant_is_caught(fn):
    with pytest.raises(AssertionError):
        _pins.check_segmented_backward(_SegBwdMutant(fn))
