"""The pages' block-wise and per-key recurrences, written out plainly in fp64.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): used to pin the
oracle's one-shot definition against the online forms the method is built on,
never by the product path.

Each function handles one head, queries q [R, d] at absolute positions
``row_index`` (default 0..R-1), keys k [N, d], values v [N, d]; the key axis is
cut into consecutive blocks whose sizes are given by ``blocks``.  The mask is
applied to each block's scores (reading notes page, section 其他算子).  A block
with no visible key for a row contributes nothing to that row.

Forms:
* ``online_normalised``: the reading-notes page, Methods, the two rescaling
  equations: l^(j+1) = e^{m^(j)-m^(j+1)} l^(j) + e^{m~ - m^(j+1)} l~ and
  O^(j+1) = diag(l^(j+1))^-1 (diag(l^(j)) e^{m^(j)-m^(j+1)} O^(j)
  + e^{m~ - m^(j+1)} P~ V_j), with m~ the block's row max, P~ = exp(S_blk - m~)
  and l~ its row sum (the plain reading of symbols the page leaves undefined).
* ``online_u_over_l``: the Polish notes, section "Nie wystarczy uśrednić...":
  state (m, l, u), both l and u rescaled by e^{m-m'} when the max grows,
  result u / l.
* ``blocked_exp_domain``: the blog, section 带在线Softmax重缩放的分块模式: the
  max is kept in the exponential domain (m = exp(row max)), l and C are
  rescaled by the ratios m^{tau-1}/m^tau and m_{[t],tau}/m^tau, and
  O = Diag(l)^-1 C at the end.
* ``per_key_recurrence``: the blog, section 递推模式: l_t = l_{t-1} + exp(k_t.q),
  a_t = a_{t-1} + v_t exp(k_t.q), o = a_L / l_L, with no max subtraction
  (valid only for small logits).
* ``blocked_no_rescale``: the blog, section 分块递推模式: ll and A accumulate raw
  exp over blocks, O = Diag(ll)^-1 A (again small logits only).
"""
from __future__ import annotations

import numpy as np


def _split(n: int, blocks):
    """Consecutive (start, stop) ranges; ``blocks`` is an int block size or a
    list of sizes summing to n."""
    if isinstance(blocks, (int, np.integer)):
        sizes = [int(blocks)] * (n // int(blocks))
        if n % int(blocks):
            sizes.append(n % int(blocks))
    else:
        sizes = [int(b) for b in blocks]
    if sum(sizes) != n or any(b <= 0 for b in sizes):
        raise ValueError("block sizes must be positive and sum to N")
    out, start = [], 0
    for b in sizes:
        out.append((start, start + b))
        start += b
    return out


def _scores(q, k, scale, causal, row_index, blocks=None):
    """Scores built block by block, the mask applied to each block's result
    (reading-notes page, section 其他算子).  Kept separate from the one-shot
    oracle's own score code so that the pins compare two computations."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.arange(q.shape[0]) if row_index is None else np.asarray(row_index)
    n = k.shape[0]
    parts = []
    for a, b in (_split(n, blocks) if blocks is not None else [(0, n)]):
        sb = scale * (q @ k[a:b].T)
        if causal:
            keys = np.arange(a, b)
            sb = np.where(keys[None, :] > rows[:, None], -np.inf, sb)
        parts.append(sb)
    return np.concatenate(parts, axis=1) if parts else np.zeros((q.shape[0], 0))


def online_normalised(q, k, v, scale, causal, blocks, row_index=None):
    """Reading-notes form: the output is kept normalised after every block.
    Returns (O, LSE) with LSE = m + ln l."""
    s = _scores(q, k, scale, causal, row_index, blocks)
    v = np.asarray(v, dtype=np.float64)
    R = s.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, v.shape[1]))
    for a, b in _split(s.shape[1], blocks):
        sb = s[:, a:b]
        m_t = np.max(sb, axis=1)                           # m~
        live = np.isfinite(m_t)
        p_t = np.exp(sb - np.where(live, m_t, 0.0)[:, None])   # P~ (0 where masked)
        l_t = p_t.sum(axis=1)                              # l~
        m_new = np.maximum(m, m_t)
        m_new_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        decay_old = np.where(np.isfinite(m), np.exp(m - m_new_safe), 0.0)
        decay_new = np.where(live, np.exp(m_t - m_new_safe), 0.0)
        l_new = decay_old * l + decay_new * l_t
        num = (l * decay_old)[:, None] * o + decay_new[:, None] * (p_t @ v[a:b])
        safe = np.where(l_new > 0, l_new, 1.0)
        o = np.where((l_new > 0)[:, None], num / safe[:, None], 0.0)
        m, l = m_new, l_new
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def online_u_over_l(q, k, v, scale, causal, blocks, row_index=None):
    """Polish-notes form: unnormalised numerator u, divided by l at the end."""
    s = _scores(q, k, scale, causal, row_index, blocks)
    v = np.asarray(v, dtype=np.float64)
    R = s.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    u = np.zeros((R, v.shape[1]))
    for a, b in _split(s.shape[1], blocks):
        sb = s[:, a:b]
        m_new = np.maximum(m, np.max(sb, axis=1))          # m'
        m_new_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        r = np.where(np.isfinite(m), np.exp(m - m_new_safe), 0.0)   # e^{m - m'}
        w = np.exp(sb - m_new_safe[:, None])               # e^{s_j - m'}
        l = r * l + w.sum(axis=1)
        u = r[:, None] * u + w @ v[a:b]
        m = m_new
    safe = np.where(l > 0, l, 1.0)
    o = np.where((l > 0)[:, None], u / safe[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(safe), -np.inf)
    return o, lse


def blocked_exp_domain(q, k, v, scale, causal, blocks, row_index=None):
    """Blog form with the running max kept as exp(row max) (multiplicative).

    Notation follows the blog: for block tau, m_{[t],tau} = exp(rowmax S_blk),
    P = Diag(m_{[t],tau})^-1 (exp(S_blk) (.) M), l_{[t],[tau]} = P 1,
    m^tau = max(m^{tau-1}, m_{[t],tau}), and
    l^tau = (m^{tau-1}/m^tau) l^{tau-1} + (m_{[t],tau}/m^tau) l_{[t],[tau]},
    C^tau = (m^{tau-1}/m^tau) C^{tau-1} + (m_{[t],tau}/m^tau) P V_tau,
    O = Diag(l^L)^-1 C^L.  Exponential-domain values overflow for logits
    beyond about 700, so this is for the small brute-force cases only.
    Returns (O, LSE) with LSE = ln(m^L) + ln(l^L).
    """
    s = _scores(q, k, scale, causal, row_index, blocks)
    v = np.asarray(v, dtype=np.float64)
    R = s.shape[0]
    m_run = np.zeros(R)          # exp(-inf): nothing seen yet
    l_run = np.zeros(R)
    c_run = np.zeros((R, v.shape[1]))
    for a, b in _split(s.shape[1], blocks):
        e = np.exp(s[:, a:b])                     # exp(S) (.) M  (masked -> 0)
        m_blk = np.exp(np.max(s[:, a:b], axis=1))  # m_{[t],tau}
        safe_blk = np.where(m_blk > 0, m_blk, 1.0)
        p = e / safe_blk[:, None]
        l_blk = p.sum(axis=1)
        m_new = np.maximum(m_run, m_blk)
        safe_new = np.where(m_new > 0, m_new, 1.0)
        r_old = m_run / safe_new
        r_blk = m_blk / safe_new
        l_run = r_old * l_run + r_blk * l_blk
        c_run = r_old[:, None] * c_run + r_blk[:, None] * (p @ v[a:b])
        m_run = m_new
    safe = np.where(l_run > 0, l_run, 1.0)
    o = np.where((l_run > 0)[:, None], c_run / safe[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(l_run > 0, np.log(np.where(m_run > 0, m_run, 1.0)) + np.log(safe), -np.inf)
    return o, lse


def per_key_recurrence(q, k, v, scale, causal, row_index=None):
    """Blog, section 递推模式: one key per step, raw exponentials, no max."""
    s = _scores(q, k, scale, causal, row_index)
    v = np.asarray(v, dtype=np.float64)
    R, N = s.shape
    l = np.zeros(R)
    a = np.zeros((R, v.shape[1]))
    for t in range(N):
        w = np.exp(s[:, t])                    # exp(k_t . q) (0 where masked)
        l = l + w
        a = a + w[:, None] * v[t][None, :]
    safe = np.where(l > 0, l, 1.0)
    o = np.where((l > 0)[:, None], a / safe[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, np.log(safe), -np.inf)
    return o, lse


def blocked_no_rescale(q, k, v, scale, causal, blocks, row_index=None):
    """Blog, section 分块递推模式: ll and A accumulate exp(S_blk) (.) M without
    any max subtraction; O = Diag(ll)^-1 A."""
    s = _scores(q, k, scale, causal, row_index, blocks)
    v = np.asarray(v, dtype=np.float64)
    R = s.shape[0]
    ll = np.zeros(R)
    A = np.zeros((R, v.shape[1]))
    for a, b in _split(s.shape[1], blocks):
        e = np.exp(s[:, a:b])
        ll = ll + e.sum(axis=1)
        A = A + e @ v[a:b]
    safe = np.where(ll > 0, ll, 1.0)
    return np.where((ll > 0)[:, None], A / safe[:, None], 0.0)


def merge_partials(o1, lse1, o2, lse2):
    """Merge two normalised partial results computed over disjoint key sets.

    This is the reading-notes rescale rule applied once to two states: with
    weights e^{LSE_p - LSE} where LSE = ln(e^{LSE_1} + e^{LSE_2}), the merged
    output is the weighted sum of the partial outputs.  (Used for the split
    key-range form of the forward pass.)
    """
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    mx = np.maximum(lse1, lse2)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - mx_safe), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - mx_safe), 0.0)
    tot = w1 + w2
    safe = np.where(tot > 0, tot, 1.0)
    o = (w1[..., None] * np.asarray(o1) + w2[..., None] * np.asarray(o2)) / safe[..., None]
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, mx_safe + np.log(safe), -np.inf)
    return o, lse
