"""Property tests of the oracle over drawn shapes, scales and score spreads
(hypothesis), each against the plain definition (oracle/brute.py) or against
another of the oracle's entry points that must give the same numbers:

* the scan is the softmax attention of every prefix (the many-to-many output
  of "Attention as an RNN", review, abstract item (3)), for scores far beyond
  e^709 and for negative scales;
* the reduction is the scan's last row, and does not depend on the order of
  the pairs ("Self-attention Does Not Need O(n^2) Memory" review, section 2:
  only the memory depends on the order);
* a packed batch is each sequence scanned on its own, zero-length sequences
  included;
* steps and appends reproduce the scan's rows (the RNN view of the review,
  abstract item (ii));
* causal self-attention row i is the scan with query q_i, full self-attention
  row i the reduction with query q_i (the review of the O(n^2) paper,
  section 2: every query in turn);
* the scan's gradients are those written out from the definition.

CPU only; each property runs a bounded number of examples."""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import brute

SETTINGS = settings(max_examples=100, deadline=None, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


def _close(got, ref, tol, what):
    err = np.max(np.abs(got - ref) / (1.0 + np.abs(ref))) if np.size(ref) else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: scaled error {err:.3e} > {tol:.1e}"


def _draw(seed, B, H, N, d, spread):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (spread * rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    return q, k, v


seeds = st.integers(0, 2 ** 32 - 1)
dims = st.sampled_from([1, 2, 3, 8, 64])
spreads = st.sampled_from([1e-3, 0.5, 1.0, 4.0, 40.0])
scales = st.sampled_from([-3.0, -0.125, 1e-3, 0.125, 1.0, 3.0])


@SETTINGS
@given(seed=seeds, B=st.integers(1, 2), H=st.integers(1, 3), N=st.integers(1, 40), d=dims,
       spread=spreads, scale=scales)
def test_scan_is_attention_over_every_prefix(seed, B, H, N, d, spread, scale):
    q, k, v = _draw(seed, B, H, N, d, spread)
    o = oracle.scan(q, k, v, scale)
    _close(o, brute.brute_scan_batch(q, k, v, scale), 1e-12, "scan vs definition")


@SETTINGS
@given(seed=seeds, H=st.integers(1, 3), N=st.integers(1, 60), d=dims, spread=spreads,
       scale=scales)
def test_reduce_is_the_last_row_and_ignores_the_order(seed, H, N, d, spread, scale):
    q, k, v = _draw(seed, 1, H, N, d, spread)
    r = oracle.reduce(q, k, v, scale)
    _close(r, oracle.scan(q, k, v, scale)[:, :, -1], 1e-13, "reduce vs last scan row")
    perm = np.random.default_rng(seed ^ 0x5A5A).permutation(N)
    rp = oracle.reduce(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                       scale)
    _close(rp, r, 1e-12, "reduce over permuted pairs")


@SETTINGS
@given(seed=seeds, lengths=st.lists(st.integers(0, 20), min_size=1, max_size=6), H=st.integers(1, 2),
       d=dims, spread=spreads)
def test_packed_sequences_are_scanned_apart(seed, lengths, H, d, spread):
    T = sum(lengths)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)).astype(np.float32)
    k = (spread * rng.standard_normal((T, H, d))).astype(np.float32)
    v = rng.standard_normal((T, H, d)).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    scale = 1.0 / math.sqrt(d)
    o = oracle.scan_segmented(q, k, v, offsets, scale)
    for a, b in zip(offsets[:-1], offsets[1:]):
        if b > a:
            kd = np.ascontiguousarray(k[a:b].transpose(1, 0, 2))[None]
            vd = np.ascontiguousarray(v[a:b].transpose(1, 0, 2))[None]
            ref = oracle.scan(q, kd, vd, scale)[0].transpose(1, 0, 2)
            _close(o[a:b], ref, 1e-13, f"sequence [{a},{b})")


@SETTINGS
@given(seed=seeds, S=st.integers(1, 3), H=st.integers(1, 2), T=st.integers(1, 24), d=dims,
       spread=spreads, scale=scales)
def test_steps_and_appends_give_the_scan_rows(seed, S, H, T, d, spread, scale):
    q, k, v = _draw(seed, S, H, T, d, spread)             # [S,H,T,d]
    ref = oracle.scan(q, k, v, scale)
    kt = np.ascontiguousarray(k.transpose(2, 0, 1, 3))     # [T,S,H,d]
    vt = np.ascontiguousarray(v.transpose(2, 0, 1, 3))
    state = oracle.state_init(S, H, d)
    for t in range(T):
        o = oracle.step(q, kt[t], vt[t], state, scale)
        _close(o, ref[:, :, t], 1e-12, f"step {t}")
    state2 = oracle.state_init(S, H, d)
    oa = oracle.append(q, kt, vt, state2, scale)
    _close(oa.transpose(1, 2, 0, 3), ref, 1e-12, "append")
    for a, b in zip(state, state2):
        assert np.array_equal(a, b)


@SETTINGS
@given(seed=seeds, H=st.integers(1, 2), N=st.integers(1, 30), d=dims, spread=spreads,
       scale=scales, causal=st.booleans())
def test_self_attention_rows_are_single_query_attention(seed, H, N, d, spread, scale, causal):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((1, H, N, d)).astype(np.float32)
    _, k, v = _draw(seed ^ 0xA5A5, 1, H, N, d, spread)
    o = oracle.self_attention(Q, k, v, scale, causal=causal)
    for i in sorted({0, N // 2, N - 1}):
        qi = np.ascontiguousarray(Q[0, :, i])
        if causal:
            ref = oracle.scan(qi, k, v, scale)[:, :, i]
        else:
            ref = oracle.reduce(qi, k, v, scale)
        _close(o[:, :, i], ref, 1e-12, f"row {i} causal={causal}")


@SETTINGS
@given(seed=seeds, B=st.integers(1, 2), H=st.integers(1, 2), N=st.integers(1, 24),
       d=st.sampled_from([1, 3, 8]), spread=spreads, scale=scales)
def test_scan_gradients_follow_the_definition(seed, B, H, N, d, spread, scale):
    q, k, v = _draw(seed, B, H, N, d, spread)
    g = np.random.default_rng(seed ^ 0x3C3C).standard_normal((B, H, N, d)).astype(np.float32)
    dq, dk, dv = oracle.scan_backward(q, k, v, g, scale)
    rq = np.zeros((H, d))
    for b in range(B):
        for h in range(H):
            gq, gk, gv = brute.brute_scan_grads(q[h], k[b, h], v[b, h], g[b, h], scale)
            rq[h] += gq
            _close(dk[b, h], gk, 1e-10, f"dK ({b},{h})")
            _close(dv[b, h], gv, 1e-10, f"dV ({b},{h})")
    _close(dq, rq, 1e-10, "dq")
