"""Plain fp64 CPU oracle for exact softmax attention (forward pass).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the bench's CPU
baseline leg use it. It shares no code with the HIP path.

What it computes is the plain definition of the method's result, with S and P
materialised in full (the very matrices the tiled GPU kernel never writes to
HBM):

* "Standard attention / forward" on the derivation blog (page "Flash
  Attention介绍", section 标准注意力 / 前向传播, the masked-forward equation):
  O = Diag((exp(QK^T) (.) M) 1)^-1 (exp(QK^T) (.) M) V, with M a causal mask or
  no mask (section 分块递推模式, first sentence).
* The reading-notes page (FlashAttention reading notes, section Background):
  S = QK^T, P = softmax(S), O = PV, per head, Q, K, V in R^{N x d}.
* The Polish notes (section "Nie wystarczy uśrednić wyników bloków"): the
  weights are normalised over all allowed keys.
* The blog's backward section (comment under 梯度推导) says the forward keeps the
  row max m and the row sum l for the backward pass; the oracle reports them as
  the natural-log logsumexp LSE_i = m_i + ln l_i.

Readings where the pages are silent (each listed in the design notes):
* a caller-supplied ``scale`` multiplies QK^T before the mask and the softmax;
* a masked pair gets weight exactly zero (logit -inf), matching the blog's
  multiplicative mask on exp(S);
* causal means key j is visible to query i iff j <= i (equal query and key
  lengths);
* grouped-query attention: query head hq reads K/V head hq // (Hq // Hkv);
* a row with no visible key (never produced by the public entry points) is
  defined as O = 0, LSE = -inf.

All arithmetic is numpy float64. Inputs are upcast exactly (bf16 and fp32
values are exactly representable in fp64).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    return a


def masked_scores(q, k, scale: float, causal: bool, row_index=None) -> np.ndarray:
    """Scaled scores S = scale * Q K^T with masked pairs set to -inf.

    q: [R, d] query rows, k: [N, d] keys. ``row_index`` gives the absolute
    position of each query row (default 0..R-1) and is used by the causal mask
    (key j visible to query i iff j <= i).  Blog page, section 分块递推模式:
    M is "a causal mask or no mask"; the reading-notes page (其他算子) applies the
    mask to the QK^T result.
    """
    q = _f64(q)
    k = _f64(k)
    s = float(scale) * (q @ k.T)
    if causal:
        rows = np.arange(q.shape[0]) if row_index is None else np.asarray(row_index)
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row-wise softmax of masked scores, with its statistics.

    Returns (P, m, l): m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i),
    P_ij = exp(S_ij - m_i) / l_i.  Rows with no visible key give P = 0,
    m = -inf, l = 0.  Polish notes, section "Nie wystarczy uśrednić...": keep
    the max m and the sum l = sum_j e^{s_j - m}; the normalised weights divide
    by l.
    """
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # masked entries: exp(-inf) = 0
    l = np.sum(e, axis=1)
    denom = np.where(empty, 1.0, l)
    p = e / denom[:, None]
    return p, m, l


def attention_head(q, k, v, scale: float, causal: bool, row_index=None):
    """One head: O = P V and LSE = m + ln l for the given query rows.

    q: [R, d], k, v: [N, d].  Returns (O [R, d], LSE [R]) in float64.
    """
    s = masked_scores(q, k, scale, causal, row_index)
    p, m, l = softmax_rows(s)
    o = p @ _f64(v)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def kv_head(hq: int, hq_total: int, hkv_total: int) -> int:
    """Grouped-query head map: contiguous groups of Hq/Hkv query heads share
    one K/V head (Polish notes, closing paragraph: GQA combines with the
    method).  Raises if Hq is not a multiple of Hkv."""
    if hkv_total <= 0 or hq_total % hkv_total != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return hq // (hq_total // hkv_total)


def attention_ref(q, k, v, causal: bool, scale: float):
    """Full oracle over [B, Hq, N, d] queries and [B, Hkv, N, d] keys/values.

    Returns (O [B, Hq, N, d], LSE [B, Hq, N]) in float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, Hq, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, hk], v[b, hk], scale, causal)
    return o, lse


def attention_rows(q, k, v, causal: bool, scale: float, rows):
    """The same definition evaluated only for selected query rows.

    ``rows`` is a sequence of (b, hq, i) triples.  Each row is computed from
    the full key set of its head exactly as in ``attention_ref`` (a row of O
    depends only on its own query row), so this is the oracle at sizes where
    materialising every N x N matrix would take too long.
    Returns (O [len(rows), d], LSE [len(rows)]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    Hq = q.shape[1]
    Hkv = k.shape[1]
    groups: dict = {}
    for n, (b, h, i) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append((n, int(i)))
    o = np.empty((len(rows), v.shape[3]), dtype=np.float64)
    lse = np.empty((len(rows),), dtype=np.float64)
    for (b, h), items in groups.items():
        idx = np.array([i for _, i in items])
        pos = np.array([n for n, _ in items])
        hk = kv_head(h, Hq, Hkv)
        ob, lb = attention_head(_f64(q[b, h, idx]), k[b, hk], v[b, hk], scale, causal,
                                row_index=idx)
        o[pos] = ob
        lse[pos] = lb
    return o, lse
