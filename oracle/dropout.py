"""Plain fp64 CPU oracle for attention with dropout on the softmax weights.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the bench's CPU baseline leg may use it; the product path never
does.  It shares no code with the HIP path; both sides implement the same
published random generator from its definition.

What the pages fix: the reading-notes page (section 其他算子) says dropout sets
entries to zero at random with some probability and that the generator's
state is kept for the backward pass; it names no generator and no scaling.
The readings taken here (each listed in the design notes):

* Dropout acts on the normalised weights P of the attention definition:
  O = (P (.) Z) V / (1 - p), with Z_ij in {0, 1} and keep probability 1 - p
  (inverted dropout, so that E[O] is the attention output).  The row
  statistics m, l and the logsumexp are those of P before dropout.
* Z comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator:
  the kept state is just (seed, offset).  Each draw is 16 bits, so one
  generator call (128 bits) serves eight keys of one query row.  For head
  unit bh = b * Hq + hq, query row i and key j = 16a + 8b + 4c + w (b and c
  in {0, 1}, w in 0..3), the draw u_ij is the 16-bit half number 4b + w,
  counting from the low half of output word 0, of the call at counter
  (2a + c, i, bh, offset) under the key (seed mod 2^32, seed // 2^32).  So
  the call at counter (2a + c, ...) serves the keys 16a + 4c + {0..3} and
  16a + 8 + 4c + {0..3}, in that order.  The pair is kept iff
  u_ij >= t = floor(p * 2^16), p being the float32 value the caller passes:
  P(keep) = 1 - t / 2^16, within 2^-16 of 1 - p.  Survivors are scaled by
  1 / (1 - p).

Gradients: with W = P (.) Z / (1 - p), O = W V, so
  dV = W^T dO,   dP = (dO V^T) (.) Z / (1 - p),
  D_i = sum_j P_ij dP_ij = dO_i . O_i,   dS = P (.) (dP - D 1^T),
  dQ = scale * dS K,   dK = scale * dS^T Q
(the blog's backward, section 反向传播, with the dropout factor in the chain).
"""
from __future__ import annotations

import numpy as np

from .attention import kv_head, masked_scores, softmax_rows

_M32 = np.uint64(0xFFFFFFFF)
# Philox4x32 constants from the generator's definition: the two round
# multipliers and the two Weyl increments of the key schedule.
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)
PHILOX_W1 = np.uint64(0xBB67AE85)
PHILOX_ROUNDS = 10


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of 32-bit counters (any shape,
    broadcast together) and a 2 x 32-bit key.  Each round multiplies
    counter words 0 and 2 by the two constants (full 64-bit products); the
    new state is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)); the key grows by the Weyl increments before every round but
    the first.  Returns the four output words as uint64 arrays < 2^32."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _M32 for x in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(PHILOX_ROUNDS):
        if r:
            k0 = (k0 + PHILOX_W0) & _M32
            k1 = (k1 + PHILOX_W1) & _M32
        p0 = PHILOX_M0 * c0          # < 2^64: no wrap in uint64
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _M32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _M32)
    return c0, c1, c2, c3


def keep_threshold(p: float) -> int:
    """t = floor(p * 2^16) for the float32 value of p (exact in fp64)."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p32 * 65536.0))


def keep_factor(p: float) -> float:
    """1 / (1 - p) for the float32 value of p, in fp64."""
    return 1.0 / (1.0 - float(np.float32(p)))


def draw_position(j):
    """For key j = 16a + 8b + 4c + w: (counter word 0 = 2a + c, 16-bit half
    index 4b + w of that call's output)."""
    j = np.asarray(j, dtype=np.int64)
    return 2 * (j >> 4) + ((j >> 2) & 1), 4 * ((j >> 3) & 1) + (j & 3)


def dropout_draws(seed: int, offset: int, bh: int, rows, n_keys: int) -> np.ndarray:
    """The 16-bit draws u_ij for the given query rows and keys 0..n_keys-1
    of head unit bh (module docstring).  Returns uint64 [len(rows), n_keys]."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    n_ctr = 2 * ((n_keys + 15) // 16)
    ctr = np.arange(n_ctr, dtype=np.int64)[None, :]
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    words = philox4x32_10(ctr, rows[:, None], int(bh), int(offset), seed & 0xFFFFFFFF, seed >> 32)
    halves = []
    for wd in words:                      # half 2m is the low half of word m
        halves += [wd & np.uint64(0xFFFF), wd >> np.uint64(16)]
    halves = np.stack(halves, axis=-1)    # [R, n_ctr, 8]
    c, hf = draw_position(np.arange(n_keys))
    return halves[:, c, hf]


def dropout_keep(seed: int, offset: int, bh: int, rows, n_keys: int, p: float) -> np.ndarray:
    """Z_ij = [u_ij >= floor(p * 2^16)] as a bool array [len(rows), n_keys]."""
    return dropout_draws(seed, offset, bh, rows, n_keys) >= np.uint64(keep_threshold(p))


def attention_dropout_head(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int,
                           bh: int, row_index=None):
    """One head with dropout: O = (P (.) Z) V / (1 - p) and the logsumexp of
    the undropped weights.  q: [R, d] (rows ``row_index``, default 0..R-1),
    k, v: [N, d].  Returns (O [R, d], LSE [R]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.arange(q.shape[0]) if row_index is None else np.asarray(row_index)
    s = masked_scores(q, k, scale, causal, rows)
    pw, m, l = softmax_rows(s)
    z = dropout_keep(seed, offset, bh, rows, s.shape[1], p)
    o = (pw * z) @ np.asarray(v, dtype=np.float64) * keep_factor(p)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def attention_dropout_ref(q, k, v, causal: bool, scale: float, p: float, seed: int, offset: int):
    """All heads: [B, Hq, N, d] queries, [B, Hkv, N, d] keys and values;
    head unit bh = b * Hq + hq.  Returns (O, LSE) in float64."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, Hq, N, v.shape[3]))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            o[b, h], lse[b, h] = attention_dropout_head(q[b, h], k[b, hk], v[b, hk], scale, causal,
                                                        p, seed, offset, b * Hq + h)
    return o, lse


def attention_dropout_rows(q, k, v, causal: bool, scale: float, p: float, seed: int, offset: int, rows):
    """Selected rows, given as (b, hq, i) triples, each from the full key set
    of its head exactly as in ``attention_dropout_ref``."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    Hq, Hkv = q.shape[1], k.shape[1]
    o = np.empty((len(rows), v.shape[3]))
    lse = np.empty((len(rows),))
    groups: dict = {}
    for n, (b, h, i) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append((n, int(i)))
    for (b, h), items in groups.items():
        idx = np.array([i for _, i in items])
        pos = np.array([n for n, _ in items])
        hk = kv_head(h, Hq, Hkv)
        o[pos], lse[pos] = attention_dropout_head(q[b, h, idx], k[b, hk], v[b, hk], scale, causal,
                                                  p, seed, offset, b * Hq + h, row_index=idx)
    return o, lse


def attention_dropout_backward_head(q, k, v, do, scale: float, causal: bool, p: float, seed: int,
                                    offset: int, bh: int):
    """Gradients (dQ, dK, dV) of one head of the dropout forward above for an
    upstream gradient dO, with every N x N matrix materialised."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n = q.shape[0]
    s = masked_scores(q, k, scale, causal)
    pw, _, _ = softmax_rows(s)
    zf = dropout_keep(seed, offset, bh, np.arange(n), n, p) * keep_factor(p)
    w = pw * zf
    o = w @ v
    dv = w.T @ do
    dp = (do @ v.T) * zf
    dsum = np.sum(do * o, axis=1)
    ds = pw * (dp - dsum[:, None])
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def attention_dropout_backward_ref(q, k, v, do, causal: bool, scale: float, p: float, seed: int,
                                   offset: int):
    """All heads; K/V gradients summed over each GQA group."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            gq, gk, gv = attention_dropout_backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], scale,
                                                         causal, p, seed, offset, b * Hq + h)
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv
