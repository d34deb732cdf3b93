"""The definition of single-query softmax attention, written out (test only).

Each function follows the plain definition and nothing else: the attention of
one query over a list of key/value pairs is the sum of the values weighted by
the softmax of the query-key scores ("Self-attention Does Not Need O(n^2)
Memory" review, section 1 Introduction); the many-to-many output of "Attention
as an RNN" (review, abstract item (3)) is that attention over every prefix.
Float64 numpy throughout, O(N^2 d): for small and moderate sizes.

The softmax subtracts the maximum score before exponentiating; that is the
usual way to evaluate a softmax and changes no value.

``combine`` and ``hillis_steele_scan`` are here only to check that the scan
result does not depend on how the prefix is bracketed. The pages name a
parallel prefix scan (and Hillis-Steele as one way to run it) but print no
combine operator; the operator below is derived: a state (m, u, w) stands for
the pair (u e^m, w e^m), and combining two states adds those pairs.
"""
from __future__ import annotations

import numpy as np


def scores(q, K, scale):
    """s_i = scale * <q, k_i> in float64. q [d], K [n,d] -> [n]."""
    return float(scale) * (np.asarray(K, np.float64) @ np.asarray(q, np.float64))


def attend(q, K, V, scale):
    """softmax(s) @ V for one query. q [d], K,V [n,d] (n >= 1) -> [d]."""
    s = scores(q, K, scale)
    p = np.exp(s - s.max())
    return (p @ np.asarray(V, np.float64)) / p.sum()


def log_normaliser(q, K, scale):
    """L = ln sum_i e^{s_i}, evaluated stably."""
    s = scores(q, K, scale)
    top = s.max()
    return top + np.log(np.exp(s - top).sum())


def brute_scan(q, K, V, scale):
    """o_k = attention of q over pairs 1..k, for every k. [n,d] -> [n,d]."""
    n = K.shape[0]
    out = np.empty((n, K.shape[1]), np.float64)
    for k in range(n):
        out[k] = attend(q, K[: k + 1], V[: k + 1], scale)
    return out


def brute_scan_batch(q, K, V, scale):
    """brute_scan over every (b,h): q [H,d], K,V [B,H,N,d] -> [B,H,N,d]."""
    B, H, N, d = K.shape
    out = np.empty((B, H, N, d), np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = brute_scan(q[h], K[b, h], V[b, h], scale)
    return out


def sdpa_scan(q, K, V, scale):
    """The same many-to-many output from torch's scaled_dot_product_attention
    on the CPU in float64: the query row repeated n times with a causal mask
    gives, in row k, attention over keys 1..k. q [d], K,V [n,d] -> [n,d]."""
    import torch
    Kt = torch.as_tensor(np.asarray(K, np.float64))
    Vt = torch.as_tensor(np.asarray(V, np.float64))
    Q = torch.as_tensor(np.asarray(q, np.float64)).expand(Kt.shape[0], -1).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(
        Q[None, None], Kt[None, None], Vt[None, None], is_causal=True, scale=float(scale))
    return out[0, 0].numpy()


def sdpa_self_attention(Q, K, V, scale, causal):
    """Self-attention (one query per token) from torch's
    scaled_dot_product_attention on the CPU in float64: Q, K, V [B,H,n,d]."""
    import torch
    Qt, Kt, Vt = (torch.as_tensor(np.asarray(x, np.float64)) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=bool(causal),
                                                           scale=float(scale))
    return out.numpy()


def softmax_reduce(q, K, V, scale):
    """Many-to-one output from torch.softmax on the CPU in float64."""
    import torch
    Kt = torch.as_tensor(np.asarray(K, np.float64))
    Vt = torch.as_tensor(np.asarray(V, np.float64))
    qt = torch.as_tensor(np.asarray(q, np.float64))
    w = torch.softmax(float(scale) * (Kt @ qt), dim=0)
    return (w @ Vt).numpy()


def brute_scan_grads(q, K, V, G, scale):
    """Gradients of the many-to-many output of one sequence, written out from
    the definition: o_k = sum_{i<=k} w_ki v_i with w_k = softmax(s_1..s_k),
    so do_k/dv_i = w_ki and do_k/ds_i = w_ki (v_i - o_k). G [n,d] holds
    dloss/do_k. Returns (dq [d], dK [n,d], dV [n,d]). O(n^2 d)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    G = np.asarray(G, np.float64)
    n = K.shape[0]
    s = scores(q, K, scale)
    dV = np.zeros_like(V)
    ds = np.zeros(n)
    for k in range(n):
        p = np.exp(s[: k + 1] - s[: k + 1].max())
        w = p / p.sum()
        o_k = w @ V[: k + 1]
        dV[: k + 1] += w[:, None] * G[k][None, :]
        ds[: k + 1] += w * ((V[: k + 1] - o_k) @ G[k])
    dK = float(scale) * ds[:, None] * q[None, :]
    dq = float(scale) * (ds @ K)
    return dq, dK, dV


def autograd_scan_grads(q, K, V, G, scale):
    """The same gradients from torch autograd through scaled_dot_product_attention
    (CPU, float64, causal, the query repeated n times)."""
    import torch
    qt = torch.tensor(np.asarray(q, np.float64), requires_grad=True)
    Kt = torch.tensor(np.asarray(K, np.float64), requires_grad=True)
    Vt = torch.tensor(np.asarray(V, np.float64), requires_grad=True)
    Q = qt.expand(Kt.shape[0], -1)
    out = torch.nn.functional.scaled_dot_product_attention(
        Q[None, None], Kt[None, None], Vt[None, None], is_causal=True, scale=float(scale))[0, 0]
    out.backward(torch.tensor(np.asarray(G, np.float64)))
    return qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy()


# ---- the combine operator (derived; see module docstring) -------------------

IDENTITY = None  # marker for the empty state


def leaf(s, v):
    """The state of a single pair: (m = s, u = 1, w = v)."""
    return (float(s), 1.0, np.asarray(v, np.float64).copy())


def combine(a, b):
    """(m_a, u_a, w_a) (+) (m_b, u_b, w_b) = (m, e^{m_a-m} u_a + e^{m_b-m} u_b,
    e^{m_a-m} w_a + e^{m_b-m} w_b) with m = max(m_a, m_b); the empty state is
    the identity."""
    if a is IDENTITY:
        return b
    if b is IDENTITY:
        return a
    ma, ua, wa = a
    mb, ub, wb = b
    m = max(ma, mb)
    fa, fb = np.exp(ma - m), np.exp(mb - m)
    return (m, fa * ua + fb * ub, fa * wa + fb * wb)


def output(state):
    """o = w / u."""
    m, u, w = state
    return w / u


def sequential_scan(leaves):
    """Inclusive scan, left to right."""
    out, acc = [], IDENTITY
    for x in leaves:
        acc = combine(acc, x)
        out.append(acc)
    return out


def hillis_steele_scan(leaves):
    """Inclusive scan by doubling rounds: in round r every position i >= 2^r
    takes (value at i - 2^r) (+) (value at i). O(n log n) combines."""
    cur = list(leaves)
    n, off = len(cur), 1
    while off < n:
        cur = [cur[i] if i < off else combine(cur[i - off], cur[i]) for i in range(n)]
        off *= 2
    return cur


def random_tree_reduce(leaves, rng):
    """Combine a list of states in a random bracketing that keeps their order."""
    items = list(leaves)
    while len(items) > 1:
        i = int(rng.integers(0, len(items) - 1))
        items[i:i + 2] = [combine(items[i], items[i + 1])]
    return items[0]
