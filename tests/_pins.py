"""Checks that pin the CPU oracle to something other than itself.

Each check takes the oracle module (or a stand-in bound to a mutated build of
it) and raises AssertionError when the oracle disagrees with the definition,
a closed form, an invariant or a library routine. test_oracle_pins.py runs
them on the real oracle; test_oracle_mutations.py runs them on builds with a
planted mistake and expects at least one to fail.
"""
from __future__ import annotations

import math
import os

import numpy as np
from scipy.special import expit, logsumexp

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.txt")


def _rows(text):
    return np.array([[float(x) for x in row.split()] for row in text.split("|")], np.float64)


def load_golden(path=GOLDEN):
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "case":
                cur = {"name": val}
                cases.append(cur)
            elif key in ("q",):
                cur[key] = np.array([float(x) for x in val.split()], np.float64)
            elif key in ("k", "v", "o", "reduce"):
                cur[key] = _rows(val)
            elif key in ("scale", "tol"):
                cur[key] = float(val)
            else:
                cur[key] = val
    return cases


def _rng(seed):
    return np.random.default_rng(seed)


def _dense(rng, B, H, N, d, spread=1.0):
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (spread * rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    return q, k, v


def _close(got, ref, tol, what):
    err = np.max(np.abs(got - ref) / (1.0 + np.abs(ref))) if np.size(ref) else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: scaled error {err:.3e} > {tol:.1e}"


# --- the definition ---------------------------------------------------------

def check_golden(orc):
    """Hand-derived closed forms (tests/golden/closed_forms.txt)."""
    for c in load_golden():
        q = c["q"].astype(np.float32)[None, :]
        k = c["k"].astype(np.float32)[None, None]
        v = c["v"].astype(np.float32)[None, None]
        if "o" in c:
            o = orc.scan(q, k, v, c["scale"])[0, 0]
            _close(o, c["o"], c["tol"], "golden " + c["name"])
        if "reduce" in c:
            r = orc.reduce(q, k, v, c["scale"])[0, 0]
            _close(r, c["reduce"][0], c["tol"], "golden reduce " + c["name"])


def check_scan_vs_definition(orc, shapes=((1, 1, 1, 1), (1, 1, 9, 3), (2, 3, 40, 64),
                                          (1, 2, 130, 128)), seed=10):
    """Oracle scan == brute-force softmax of every prefix == torch SDPA (causal,
    repeated query), float64, for scale 1/sqrt(d) and a spread that takes
    scores far beyond e^709."""
    rng = _rng(seed)
    for (B, H, N, d) in shapes:
        for spread, scale in ((1.0, 1.0 / math.sqrt(d)), (30.0, 3.0)):
            q, k, v = _dense(rng, B, H, N, d, spread)
            o = orc.scan(q, k, v, scale)
            ref = brute.brute_scan_batch(q, k, v, scale)
            _close(o, ref, 1e-12, f"scan vs brute {B,H,N,d} spread {spread}")
            sd = brute.sdpa_scan(q[0], k[0, 0], v[0, 0], scale)
            _close(o[0, 0], sd, 1e-12, f"scan vs sdpa {B,H,N,d}")


def check_stats(orc, seed=11):
    """Running max == numpy maximum.accumulate of the scores; L = m + ln u ==
    scipy logsumexp of the prefix scores."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 1, 2, 60, 16, spread=5.0)
    scale = 0.25
    _, m, lse = orc.scan(q, k, v, scale, stats=True)
    for h in range(2):
        s = brute.scores(q[h], k[0, h], scale)
        np.testing.assert_allclose(m[0, h], np.maximum.accumulate(s), rtol=1e-14, atol=1e-14)
        ref = np.array([logsumexp(s[: i + 1]) for i in range(s.size)])
        _close(lse[0, h], ref, 1e-13, "log-normaliser")


def check_single_token(orc, seed=12):
    """o_1 = v_1 exactly (u = 1, w = v_1)."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 3, 2, 1, 64, spread=10.0)
    o = orc.scan(q, k, v, 0.125)
    assert np.array_equal(o, v.astype(np.float64)), "o_1 != v_1"


def check_running_mean(orc, seed=13):
    """q = 0: every score is 0 and o_k is the mean of v_1..v_k."""
    rng = _rng(seed)
    _, k, v = _dense(rng, 2, 2, 100, 8)
    q = np.zeros((2, 8), np.float32)
    o = orc.scan(q, k, v, 0.5)
    ref = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 101)[None, None, :, None]
    _close(o, ref, 1e-14, "running mean")


def check_two_tokens(orc, seed=14):
    """o_2 = expit(s_1 - s_2) v_1 + expit(s_2 - s_1) v_2."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 1, 1, 2, 32, spread=3.0)
    scale = 0.3
    s = brute.scores(q[0], k[0, 0], scale)
    ref = expit(s[0] - s[1]) * v[0, 0, 0] + expit(s[1] - s[0]) * v[0, 0, 1]
    o = orc.scan(q, k, v, scale)
    _close(o[0, 0, 1], ref, 1e-14, "two-token logistic")


def check_dominating_key(orc, seed=15):
    """A key whose score exceeds every other by > 40 takes the whole weight
    from its position on; earlier outputs do not see it."""
    rng = _rng(seed)
    d, N, j = 4, 50, 20
    q = np.array([[1, 0, 0, 0]], np.float32)
    k = rng.uniform(-1, 1, (1, 1, N, d)).astype(np.float32)
    k[0, 0, j, 0] = 60.0
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    o = orc.scan(q, k, v, 1.0)
    _close(o[0, 0, j:], np.broadcast_to(v[0, 0, j].astype(np.float64), (N - j, d)), 1e-15,
           "dominating key")
    ref = brute.brute_scan(q[0], k[0, 0, :j], v[0, 0, :j], 1.0)
    _close(o[0, 0, :j], ref, 1e-13, "before the dominating key")


def check_shift_invariance(orc, seed=16):
    """Adding c to every score changes nothing, for c = +-1000 (far past the
    range of exp): realised with an extra coordinate q' = (q, 1), k' = (k, c)."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 1, 1, 80, 7)
    base = orc.scan(q, k, v, 1.0)
    v2 = np.concatenate([v, np.zeros((1, 1, 80, 1), np.float32)], axis=3)
    for c in (-1000.0, 1000.0):
        q2 = np.concatenate([q, np.ones((1, 1), np.float32)], axis=1)
        k2 = np.concatenate([k, np.full((1, 1, 80, 1), c, np.float32)], axis=3)
        o2 = orc.scan(q2, k2, v2, 1.0)
        _close(o2[..., :7], base, 1e-12, f"shift by {c}")
        assert np.all(o2[..., 7] == 0.0)


def check_convex_hull(orc, seed=17):
    """Each output coordinate lies between the min and max of the values seen."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 2, 2, 200, 16, spread=4.0)
    o = orc.scan(q, k, v, 0.25)
    lo = np.minimum.accumulate(v.astype(np.float64), axis=2)
    hi = np.maximum.accumulate(v.astype(np.float64), axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12), "outside the convex hull"


# --- combine order ----------------------------------------------------------

def check_bracketing(orc, seed=18):
    """The derived combine is associative: sequential order, Hillis-Steele
    order (the scan the Aaren review names) and random bracketings agree, and
    agree with the oracle's scan."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 1, 1, 37, 5, spread=6.0)
    scale = 0.7
    s = brute.scores(q[0], k[0, 0], scale)
    leaves = [brute.leaf(si, vi) for si, vi in zip(s, v[0, 0])]
    seq = np.array([brute.output(x) for x in brute.sequential_scan(leaves)])
    hs = np.array([brute.output(x) for x in brute.hillis_steele_scan(leaves)])
    _close(hs, seq, 1e-13, "Hillis-Steele vs sequential")
    for t in range(5):
        tr = brute.output(brute.random_tree_reduce(leaves, rng))
        _close(tr, seq[-1], 1e-13, "random bracketing")
    _close(orc.scan(q, k, v, scale)[0, 0], seq, 1e-12, "oracle vs combine scan")
    for t in range(20):
        a, b, c = (brute.leaf(rng.normal(0, 20), rng.standard_normal(3)) for _ in range(3))
        l = brute.combine(brute.combine(a, b), c)
        r = brute.combine(a, brute.combine(b, c))
        assert abs(l[0] - r[0]) == 0
        _close(np.append(l[2], l[1]), np.append(r[2], r[1]), 1e-13, "associativity")


# --- many-to-one, step, segmented -------------------------------------------

def check_reduce(orc, seed=19):
    """Reduce == last scan row == torch softmax @ V, and does not depend on
    the order of the pairs (only the memory needed does, per section 2 of the
    memory-efficient-attention review)."""
    rng = _rng(seed)
    q, k, v = _dense(rng, 2, 3, 257, 16, spread=3.0)
    scale = 0.25
    r, m, lse = orc.reduce(q, k, v, scale, stats=True)
    o = orc.scan(q, k, v, scale)
    _close(r, o[:, :, -1], 1e-14, "reduce vs last scan row")
    for b in range(2):
        for h in range(3):
            _close(r[b, h], brute.softmax_reduce(q[h], k[b, h], v[b, h], scale), 1e-12,
                   "reduce vs softmax")
            s = brute.scores(q[h], k[b, h], scale)
            assert abs(m[b, h] - s.max()) <= 1e-13 * (1 + abs(s.max()))
            _close(lse[b, h], logsumexp(s), 1e-13, "reduce log-normaliser")
    perm = rng.permutation(257)
    rp = orc.reduce(q, k[:, :, perm], v[:, :, perm], scale)
    _close(rp, r, 1e-13, "reduce permutation")


def check_step(orc, seed=20):
    """t single-pair updates from the empty state give the scan of those t
    pairs; saving the state and resuming gives the same as not stopping."""
    rng = _rng(seed)
    S, H, d, T = 5, 2, 16, 30
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (2 * rng.standard_normal((T, S, H, d))).astype(np.float32)
    v = rng.standard_normal((T, S, H, d)).astype(np.float32)
    scale = 0.25
    st = orc.state_init(S, H, d)
    outs, saved = [], None
    for t in range(T):
        outs.append(orc.step(q, k[t], v[t], st, scale))
        if t == 11:
            saved = tuple(a.copy() for a in st)
    outs = np.stack(outs)                                  # [T,S,H,d]
    ref = brute.brute_scan_batch(q, k.transpose(1, 2, 0, 3), v.transpose(1, 2, 0, 3), scale)
    _close(outs.transpose(1, 2, 0, 3), ref, 1e-12, "steps vs brute scan")
    s_all = np.stack([[brute.scores(q[h], k[:, s, h], scale) for h in range(H)] for s in range(S)])
    _close(st[0] + np.log(st[1]), logsumexp(s_all, axis=-1), 1e-13, "step log-normaliser")
    resumed = tuple(a.copy() for a in saved)
    for t in range(12, T):
        o = orc.step(q, k[t], v[t], resumed, scale)
    assert np.array_equal(o, outs[-1]) and all(np.array_equal(a, b) for a, b in zip(resumed, st))


def check_append(orc, seed=25):
    """Appending tokens in blocks of any size continues the same scan: from a
    state that already holds a prefix, each appended token's output and the
    final log-normaliser equal brute force over prefix + appended tokens
    (sizes S, H, T, d all distinct so a swapped axis shows)."""
    rng = _rng(seed)
    S, H, d, T0, T1 = 4, 3, 8, 7, 11
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (2 * rng.standard_normal((T0 + T1, S, H, d))).astype(np.float32)
    v = rng.standard_normal((T0 + T1, S, H, d)).astype(np.float32)
    scale = 0.3
    st = orc.state_init(S, H, d)
    first = orc.append(q, k[:T0], v[:T0], st, scale)
    second = orc.append(q, k[T0:], v[T0:], st, scale)
    assert first.shape == (T0, S, H, d) and second.shape == (T1, S, H, d)
    ref = brute.brute_scan_batch(q, k.transpose(1, 2, 0, 3), v.transpose(1, 2, 0, 3), scale)
    got = np.concatenate([first, second]).transpose(1, 2, 0, 3)      # [S,H,T,d]
    _close(got, ref, 1e-12, "blocked appends vs brute scan")
    s_all = np.stack([[brute.scores(q[h], k[:, s, h], scale) for h in range(H)] for s in range(S)])
    _close(st[0] + np.log(st[1]), logsumexp(s_all, axis=-1), 1e-13, "append log-normaliser")
    _close(st[0], s_all.max(axis=-1), 1e-13, "m is the running maximum of the scores")
    empty = orc.append(q, k[:0], v[:0], st, scale)
    assert empty.shape == (0, S, H, d)


def check_self_attention(orc, seed=26):
    """One query per token: every row equals brute-force attention of its own
    query over its prefix (causal) or over all pairs, and torch SDPA in
    float64; with every query equal to q_h the causal rows are the scan and
    the full rows the reduction; a row range is the slice of the whole."""
    rng = _rng(seed)
    B, H, N, d = 2, 3, 37, 8
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    k = (1.5 * k).astype(np.float32)
    scale = 0.4
    for causal in (True, False):
        o, lse = orc.self_attention(q, k, v, scale, causal=causal, stats=True)
        _close(o, brute.sdpa_self_attention(q, k, v, scale, causal), 1e-12, "vs torch SDPA")
        for b, h, i in ((0, 0, 0), (1, 2, N - 1), (0, 1, 17), (1, 0, 5)):
            last = i + 1 if causal else N
            _close(o[b, h, i], brute.attend(q[b, h, i], k[b, h, :last], v[b, h, :last], scale),
                   1e-12, "vs brute force")
            _close(lse[b, h, i], brute.log_normaliser(q[b, h, i], k[b, h, :last], scale), 1e-13,
                   "self-attention log-normaliser")
        part = orc.self_attention(q, k, v, scale, causal=causal, rows=(10, 23))
        _close(part, o[:, :, 10:23], 1e-15, "row range")
    qh = rng.standard_normal((H, d)).astype(np.float32)
    same = np.ascontiguousarray(np.broadcast_to(qh[None, :, None, :], (B, H, N, d)))
    _close(orc.self_attention(same, k, v, scale, causal=True), orc.scan(qh, k, v, scale), 1e-13,
           "equal queries, causal == scan")
    full = orc.self_attention(same, k, v, scale, causal=False)
    _close(full, np.broadcast_to(orc.reduce(qh, k, v, scale)[:, :, None, :], full.shape), 1e-13,
           "equal queries, all pairs == reduce")


def check_bf16_round(orc, seed=27):
    """Round-to-nearest-even to 8 significant bits: hand-checked ties and
    neighbours, and torch's own float32 -> bfloat16 conversion on random
    float32 values."""
    import torch
    one = 1.0
    cases = {one + 2 ** -8: one, one + 3 * 2 ** -8: one + 2 ** -6, one + 2 ** -9: one,
             one + 2 ** -8 + 2 ** -20: one + 2 ** -7, -(one + 2 ** -7 + 2 ** -8): -(one + 2 ** -6),
             0.0: 0.0, 3.0: 3.0, 2 ** -100 * 1.00390625: 2 ** -100}
    for a, want in cases.items():
        assert orc.bf16_round(a) == want, (a, orc.bf16_round(a), want)
    r = (_rng(seed).standard_normal(10000) * 10.0).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_round(r), ref)


def check_scan_f64(orc, seed=30):
    """The float64-input scan: against brute force on keys and values that
    are not float32 values (a spread of ±200 in the scores included), and
    equal to the float32-input scan where the inputs are float32 values."""
    rng = _rng(seed)
    B, H, N, d = 2, 3, 37, 5
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((B, H, N, d)) * (1 + np.arange(N)[:, None] * 2.0)
    v = rng.standard_normal((B, H, N, d)) / 3.0
    o = orc.scan_f64(q, k, v, 0.7)
    _close(o, brute.brute_scan_batch(q, k, v, 0.7), 1e-12, "float64 scan vs brute force")
    q32, k32, v32 = (a.astype(np.float32) for a in (q, k, v))
    _close(orc.scan_f64(q32.astype(np.float64), k32.astype(np.float64), v32.astype(np.float64), 0.7),
           orc.scan(q32, k32, v32, 0.7), 1e-14, "float64 scan == float32-input scan")


def check_layer(orc, seed=28):
    """The layer is the projection followed by the scan: per (b, h), brute
    force over k = x W_K[:, h], v = x W_V[:, h] (written out here with its own
    indexing, in float64), the output rounded to bf16 or not."""
    rng = _rng(seed)
    B, N, Dm, H, d = 2, 9, 5, 3, 4
    x = rng.standard_normal((B, N, Dm)).astype(np.float32)
    w = (rng.standard_normal((Dm, 2 * H * d)) / 2).astype(np.float32)
    q = rng.standard_normal((H, d)).astype(np.float32)
    scale = 0.5
    o = orc.layer_forward(x, w, q, scale, out_bf16=False)
    assert o.shape == (B, N, H, d)
    for b in range(B):
        for h in range(H):
            kh = np.einsum("nm,mj->nj", x[b].astype(np.float64), w[:, h * d:(h + 1) * d])
            vh = np.einsum("nm,mj->nj", x[b].astype(np.float64), w[:, (H + h) * d:(H + h + 1) * d])
            ref = brute.brute_scan(q[h], kh, vh, scale)
            _close(o[b, :, h], ref, 1e-12, "layer vs projection + brute scan")
    ob = orc.layer_forward(x, w, q, scale, out_bf16=True)
    assert np.array_equal(ob, orc.bf16_round(o))


def check_mean_query(orc, seed=29):
    """Mean-query attention: torch's mean and softmax in float64 give the
    same; equal query rows make it the plain reduction with that query; the
    token order does not matter."""
    import torch
    rng = _rng(seed)
    B, H, N, d = 2, 3, 41, 8
    hq, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    scale = 0.6
    o, g = orc.mean_query_attention(hq, k, v, scale, stats=True)
    gt = torch.from_numpy(hq).double().mean(dim=2)
    w = torch.softmax(scale * torch.einsum("bhnd,bhd->bhn", torch.from_numpy(k).double(), gt), dim=-1)
    ref = torch.einsum("bhn,bhnd->bhd", w, torch.from_numpy(v).double()).numpy()
    _close(o, ref, 1e-12, "mean query vs torch")
    assert np.allclose(g, gt.numpy(), rtol=1e-15, atol=0)
    qh = rng.standard_normal((H, d)).astype(np.float32)
    same = np.ascontiguousarray(np.broadcast_to(qh[None, :, None, :], (B, H, N, d)))
    _close(orc.mean_query_attention(same, k, v, scale), orc.reduce(qh, k, v, scale), 1e-13,
           "equal query rows == reduce")
    perm = rng.permutation(N)
    _close(orc.mean_query_attention(hq[:, :, perm], k[:, :, perm], v[:, :, perm], scale), o,
           1e-12, "token order")


def check_segmented(orc, seed=21):
    """Each packed sequence is scanned on its own: == brute force per segment;
    empty and length-1 segments included."""
    rng = _rng(seed)
    lengths = np.array([1, 0, 5, 1, 17, 0, 0, 64, 3, 1], np.int64)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(offs[-1]), 3, 8
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (2 * rng.standard_normal((T, H, d))).astype(np.float32)
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    scale = 0.35
    o, m, lse = orc.scan_segmented(q, k, v, offs, scale, stats=True)
    for sidx in range(lengths.size):
        a, b = offs[sidx], offs[sidx + 1]
        for h in range(H):
            if b > a:
                ref = brute.brute_scan(q[h], k[a:b, h], v[a:b, h], scale)
                _close(o[a:b, h], ref, 1e-12, f"segment {sidx} head {h}")
                s = brute.scores(q[h], k[a:b, h], scale)
                _close(lse[a:b, h], [logsumexp(s[: i + 1]) for i in range(b - a)], 1e-13,
                       "segment log-normaliser")
    one = offs[:-1][lengths == 1]
    assert np.array_equal(o[one], v[one].astype(np.float64)), "length-1 segment"


# --- gradients ---------------------------------------------------------------

def check_backward(orc, seed=22):
    """The oracle's gradients (reverse recurrence) == the definition written
    out (brute force) == torch autograd through SDPA, float64, including a
    spread that takes scores far past the range of exp; dq sums over the batch."""
    rng = _rng(seed)
    for (B, H, N, d, spread, scale) in ((2, 2, 40, 6, 1.0, 0.4), (1, 3, 70, 16, 25.0, 2.0),
                                        (2, 1, 1, 4, 1.0, 1.0)):
        q = rng.standard_normal((H, d)).astype(np.float32)
        k = (spread * rng.standard_normal((B, H, N, d))).astype(np.float32)
        v = rng.standard_normal((B, H, N, d)).astype(np.float32)
        g = rng.standard_normal((B, H, N, d)).astype(np.float32)
        dq, dk, dv = orc.scan_backward(q, k, v, g, scale)
        for h in range(H):
            acc = np.zeros(d)
            for b in range(B):
                bq, bk, bv = brute.brute_scan_grads(q[h], k[b, h], v[b, h], g[b, h], scale)
                aq, ak, av = brute.autograd_scan_grads(q[h], k[b, h], v[b, h], g[b, h], scale)
                _close(dk[b, h], bk, 1e-11, "dk vs definition")
                _close(dv[b, h], bv, 1e-11, "dv vs definition")
                _close(bk, ak, 1e-11, "dk definition vs autograd")
                _close(bv, av, 1e-11, "dv definition vs autograd")
                _close(bq, aq, 1e-11, "dq definition vs autograd")
                acc += bq
            _close(dq[h], acc, 1e-11, "dq (batch sum) vs definition")


def check_segmented_backward(orc, seed=30):
    """Packed gradients == torch autograd through a packed forward written
    out here (a softmax over each sequence's prefix, sequence by sequence),
    with empty, length-1 and longer sequences; dq adds all sequences."""
    import torch
    rng = _rng(seed)
    lengths = np.array([3, 0, 1, 17, 0, 9, 1], np.int64)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d, scale = int(offs[-1]), 2, 5, 0.7
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (2 * rng.standard_normal((T, H, d))).astype(np.float32)
    v, g = (rng.standard_normal((T, H, d)).astype(np.float32) for _ in range(2))
    dq, dk, dv = orc.scan_segmented_backward(q, k, v, g, offs, scale)
    qt, kt, vt = (torch.tensor(x.astype(np.float64), requires_grad=True) for x in (q, k, v))
    rows = []
    for t in range(T):
        a = int(offs[np.searchsorted(offs, t, side="right") - 1])
        s_ = scale * (kt[a:t + 1] * qt[None]).sum(-1)          # [len, H]
        w = torch.softmax(s_, dim=0)
        rows.append((w[..., None] * vt[a:t + 1]).sum(0))       # [H, d]
    torch.stack(rows).backward(torch.tensor(g.astype(np.float64)))
    _close(dk, kt.grad.numpy(), 1e-11, "packed dk vs autograd")
    _close(dv, vt.grad.numpy(), 1e-11, "packed dv vs autograd")
    _close(dq, qt.grad.numpy(), 1e-11, "packed dq vs autograd")


def check_backward_finite_differences(orc, seed=23):
    """Central differences of loss = sum(g * o) through the forward oracle."""
    rng = _rng(seed)
    B, H, N, d, scale = 1, 1, 5, 3, 0.7
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    g = rng.standard_normal((B, H, N, d))
    dq, dk, dv = orc.scan_backward(*(x.astype(np.float32) for x in (q, k, v, g)), scale)
    # finite differences need inputs exactly representable in float32
    q, k, v, g = (x.astype(np.float32).astype(np.float64) for x in (q, k, v, g))

    def loss(q_, k_, v_):
        o = orc.scan(q_.astype(np.float32), k_.astype(np.float32), v_.astype(np.float32), scale)
        return float((o * g).sum())
    h = 2.0 ** -10  # exact in float32 for these magnitudes
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.reshape(-1)
        for i in range(0, flat.size, max(1, flat.size // 7)):
            old = flat[i]
            flat[i] = old + h
            lp = loss(q, k, v)
            flat[i] = old - h
            lm = loss(q, k, v)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad.reshape(-1)[i]) <= 1e-5 * (1 + abs(fd)), (name, i, fd)


def check_backward_closed_forms(orc, seed=24):
    """One pair: o_1 = v_1, so dv_1 = g_1 and the score gradient is 0. Equal
    scores (q = 0): dv_i = sum_{k>=i} g_k / k."""
    rng = _rng(seed)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    k = rng.standard_normal((3, 2, 1, 8)).astype(np.float32)
    v = rng.standard_normal((3, 2, 1, 8)).astype(np.float32)
    g = rng.standard_normal((3, 2, 1, 8)).astype(np.float32)
    dq, dk, dv = orc.scan_backward(q, k, v, g, 0.3)
    assert np.array_equal(dv, g.astype(np.float64)), "dv_1 != g_1"
    assert np.all(np.abs(dk) <= 1e-15) and np.all(np.abs(dq) <= 1e-14), "single pair: ds != 0"
    N = 50
    k = rng.standard_normal((1, 1, N, 4)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, 4)).astype(np.float32)
    g = rng.standard_normal((1, 1, N, 4)).astype(np.float32)
    _, _, dv = orc.scan_backward(np.zeros((1, 4), np.float32), k, v, g, 1.0)
    ref = np.cumsum((g[0, 0].astype(np.float64) / np.arange(1, N + 1)[:, None])[::-1], axis=0)[::-1]
    _close(dv[0, 0], ref, 1e-13, "equal-score dv")


ALL = [check_golden, check_scan_vs_definition, check_stats, check_single_token,
       check_running_mean, check_two_tokens, check_dominating_key, check_shift_invariance,
       check_convex_hull, check_bracketing, check_reduce, check_step, check_append, check_self_attention, check_bf16_round, check_scan_f64, check_layer, check_mean_query, check_segmented,
       check_backward, check_segmented_backward, check_backward_finite_differences, check_backward_closed_forms]
