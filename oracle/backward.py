"""Plain fp64 CPU oracle for the gradients of exact softmax attention.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the bench's CPU baseline leg may use it; the product path never
does.  It shares no code with the HIP path.

What it computes is the plain definition, with S, P, dP and dS materialised in
full.  The derivation blog (page "Flash Attention介绍", section 反向传播, the
standard attention backward) gives, for O = Diag(E 1)^-1 E V with
E = exp(Q K^T) (.) M:

    dV = P^T dO                                 (P = Diag(E 1)^-1 E)
    dE (.) E = P (.) (dO V^T - diag(dO O^T) 1^T)
    dQ = (dE (.) E) K,   dK = (dE (.) E)^T Q

With the softmax scale of the forward (S = scale * Q K^T), the chain rule
multiplies dQ and dK by scale.  Writing D_i = sum_d dO_id O_id (the
diag(dO O^T) term), dP = dO V^T and dS = P (.) (dP - D 1^T):

    dV = P^T dO,   dQ = scale * dS K,   dK = scale * dS^T Q.

Grouped-query attention: K/V head hk serves the query heads of its group, so
its dK and dV are the sums over those heads.

``backward_blocked`` is the blog's FlashAttention backward (section
Flash Attention 反向传播, 梯度推导): P of each (query block, key block) pair is
recomputed from the stored row statistics, and each pair adds its share to
dV, dQ and dK.  It exists only to pin ``attention_backward_head``: the two
must agree to rounding.
"""
from __future__ import annotations

import numpy as np

from .attention import kv_head, masked_scores, softmax_rows


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_backward_head(q, k, v, do, scale: float, causal: bool, return_ds: bool = False):
    """Gradients of one head: returns (dQ [N, d], dK [N, d], dV [N, d]) for
    O = softmax(scale Q K^T, masked) V and an upstream gradient dO, and with
    ``return_ds`` also dS [N, N].  Rows with no visible key contribute
    nothing."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    s = masked_scores(q, k, scale, causal)
    p, _, _ = softmax_rows(s)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(do * o, axis=1)              # D_i = diag(dO O^T)
    ds = p * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    if return_ds:
        return dq, dk, dv, ds
    return dq, dk, dv


def attention_backward_ref(q, k, v, do, causal: bool, scale: float):
    """Gradients over [B, Hq, N, d] queries / dO and [B, Hkv, N, d] keys and
    values.  Returns (dQ, dK, dV) in float64, dK and dV summed over each
    GQA group."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            gq, gk, gv = attention_backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal)
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv


def backward_blocked(q, k, v, do, scale: float, causal: bool, bq: int, bk: int):
    """The blog's FlashAttention backward for one head, with query blocks of
    bq rows and key blocks of bk rows: the forward's row statistics are kept
    as LSE = m + ln l, and every block pair recomputes its P from them
    (P_ij = exp(S_ij - LSE_i)), then adds P^T dO to dV, dS K to dQ and
    dS^T Q to dK (both times scale), with dS = P (.) (dO V^T - D)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    # forward statistics, kept per row (what the forward stores)
    s_full = masked_scores(q, k, scale, causal)
    p_full, m, l = softmax_rows(s_full)
    o = p_full @ v
    lse = m + np.log(l)
    dsum = np.sum(do * o, axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for t0 in range(0, n, bq):
        rows = np.arange(t0, min(n, t0 + bq))
        for u0 in range(0, n, bk):
            cols = np.arange(u0, min(n, u0 + bk))
            s = float(scale) * (q[rows] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            p = np.exp(s - lse[rows][:, None])
            dv[cols] += p.T @ do[rows]
            dp = do[rows] @ v[cols].T
            ds = p * (dp - dsum[rows][:, None])
            dq[rows] += float(scale) * (ds @ k[cols])
            dk[cols] += float(scale) * (ds.T @ q[rows])
    return dq, dk, dv
