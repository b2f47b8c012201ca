"""Pins of the dropout oracle (oracle/dropout.py) to things other than itself.

* The generator: Philox4x32-10's published known-answer vectors
  (tests/golden/philox4x32_10_kat.json), and the statistics uniform 16-bit
  draws must show (keep rate 1 - p, independent streams per head, offset
  and seed).
* The keep mask: each element is the draw of its own counter, checked one
  element at a time against single generator calls.
* The forward: p = 0 gives the attention oracle; the logsumexp does not see
  dropout; the mean over many seeds is the attention output (inverted
  dropout); with Q = 0 and V = 1 each row is its kept-key count over
  (visible keys) (1 - p).
* The backward: finite differences of the dropout forward (the mask is a
  fixed function of the seed), torch's fp64 autograd through an explicit
  mask, and p = 0 gives the backward oracle.
Planted-mistake copies must fail at least one pin each.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.attention import attention_head, masked_scores, softmax_rows
from oracle.backward import attention_backward_head
from oracle.dropout import (attention_dropout_backward_head, attention_dropout_backward_ref,
                            attention_dropout_head, attention_dropout_ref, attention_dropout_rows,
                            draw_position, dropout_draws, dropout_keep, keep_factor, keep_threshold,
                            philox4x32_10)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# ---- the generator -----------------------------------------------------------

def test_philox_known_answer_vectors():
    with open(GOLDEN) as f:
        kat = json.load(f)
    assert len(kat["vectors"]) == 3
    for vec in kat["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        out = philox4x32_10(*c, *k)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["output"]]


def test_philox_vectorised_equals_elementwise():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2**32, size=(4, 37), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    batch = philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for n in range(37):
        one = philox4x32_10(int(c[0, n]), int(c[1, n]), int(c[2, n]), int(c[3, n]), k0, k1)
        for w in range(4):
            assert int(batch[w][n]) == int(one[w])


def test_threshold_and_factor():
    assert keep_threshold(0.0) == 0
    assert keep_threshold(0.5) == 2**15
    assert keep_threshold(0.25) == 2**14
    p32 = float(np.float32(0.1))
    assert keep_threshold(0.1) == int(np.floor(p32 * 2**16)) == 6553
    assert keep_factor(0.5) == 2.0
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        with pytest.raises(ValueError):
            keep_threshold(bad)


def test_draw_positions_cover_each_call_once():
    """Every call (counter) serves exactly eight keys, one per 16-bit half:
    keys 16a + 4c + {0..3} and 16a + 8 + 4c + {0..3}, in that order."""
    j = np.arange(64)
    c, hf = draw_position(j)
    for ctr in range(8):
        keys = j[c == ctr]
        a, cc = ctr // 2, ctr % 2
        want = [16 * a + 4 * cc + w for w in range(4)] + [16 * a + 8 + 4 * cc + w for w in range(4)]
        assert list(keys) == want
        assert list(hf[c == ctr]) == list(range(8))


# ---- pins of the keep mask -----------------------------------------------------

def pin_keep_elementwise(keep):
    """Each Z_ij is [u_ij >= t] with u_ij the 16-bit half 4b + w of the call
    at counter (2a + c, i, bh, offset), for j = 16a + 8b + 4c + w."""
    rng = np.random.default_rng(2)
    for seed, offset, bh, p in [(0, 0, 0, 0.5), (2**40 + 77, 3, 5, 0.1), (123456789, 9, 1000, 0.9)]:
        z = keep(seed, offset, bh, np.arange(40), 45, p)
        t = keep_threshold(p)
        for _ in range(80):
            i, j = int(rng.integers(0, 40)), int(rng.integers(0, 45))
            a, b, c, w = j // 16, (j // 8) % 2, (j // 4) % 2, j % 4
            half = 4 * b + w
            word = philox4x32_10(2 * a + c, i, bh, offset, seed & 0xFFFFFFFF, seed >> 32)[half // 2]
            u = (int(word) >> (16 * (half % 2))) & 0xFFFF
            assert bool(z[i, j]) == (u >= t), (seed, offset, bh, i, j)


def pin_keep_rate(keep):
    """A uniform 16-bit draw passes u >= floor(p 2^16) with probability
    within 2^-16 of 1 - p: the kept fraction of 65536 draws is within
    5 sigma of it."""
    for p in (0.1, 0.5, 0.9):
        z = keep(7, 1, 3, np.arange(256), 256, p)
        n = z.size
        assert abs(z.mean() - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / n), p


def pin_streams_independent(keep):
    """Different heads, offsets or seeds give unrelated masks: two masks at
    p = 0.5 agree on about half of the elements, not on all."""
    base = keep(11, 0, 0, np.arange(128), 128, 0.5)
    for other in (keep(11, 0, 1, np.arange(128), 128, 0.5), keep(11, 1, 0, np.arange(128), 128, 0.5),
                  keep(12, 0, 0, np.arange(128), 128, 0.5), keep(11 + 2**32, 0, 0, np.arange(128), 128, 0.5)):
        agree = np.mean(base == other)
        assert abs(agree - 0.5) <= 5 * np.sqrt(0.25 / base.size), agree


def test_draws_are_uniform():
    """The top 4 bits of 2^16 16-bit draws fill 16 bins evenly (chi-square,
    15 degrees of freedom, below the 0.1% point 37.7), and so do the low 4."""
    u = dropout_draws(5, 2, 9, np.arange(256), 256)
    assert int(u.max()) < 2**16
    for bits in (u >> np.uint64(12), u & np.uint64(15)):
        hist = np.bincount(bits.astype(np.int64).ravel(), minlength=16)
        e = u.size / 16
        assert np.sum((hist - e) ** 2 / e) < 37.7


# ---- pins of the forward -------------------------------------------------------

def pin_p_zero(fwd):
    """p = 0 keeps every element with factor 1: the attention oracle."""
    for causal in (False, True):
        q, k, v = (_rand((9, 4), 10 + i) for i in range(3))
        o, lse = fwd(q, k, v, 0.6, causal, 0.0, 5, 0, 2)
        o0, lse0 = attention_head(q, k, v, 0.6, causal)
        assert np.max(np.abs(o - o0)) <= 1e-15 and np.max(np.abs(lse - lse0)) <= 1e-15


def pin_lse_undropped(fwd):
    """The logsumexp is a statistic of the scores, before dropout."""
    for causal in (False, True):
        q, k, v = (_rand((11, 3), 20 + i) for i in range(3))
        _, lse = fwd(q, k, v, 0.9, causal, 0.3, 17, 4, 1)
        _, lse0 = attention_head(q, k, v, 0.9, causal)
        assert np.max(np.abs(lse - lse0)) <= 1e-12


def pin_expectation(fwd):
    """Inverted dropout is unbiased: the mean of O over many seeds is the
    attention output, within 6 standard errors."""
    n, d, p, reps = 6, 2, 0.3, 3000
    for causal in (False, True):
        q, k, v = (_rand((n, d), 30 + i) for i in range(3))
        o0, _ = attention_head(q, k, v, 0.8, causal)
        outs = np.stack([fwd(q, k, v, 0.8, causal, p, s, 0, 0)[0] for s in range(reps)])
        se = outs.std(axis=0) / np.sqrt(reps)
        assert np.all(np.abs(outs.mean(axis=0) - o0) <= 6 * se + 1e-12), causal


def pin_counts(fwd):
    """Q = 0 makes the weights uniform over the visible keys and V = 1 makes
    each row sum its kept weights: O_i = (#kept visible keys of row i) /
    (#visible keys * (1 - p)), with the kept keys read from the mask."""
    n, d, p, seed, offset, bh = 13, 3, 0.4, 99, 2, 6
    q, k, v = np.zeros((n, d)), _rand((n, d), 40), np.ones((n, d))
    z = dropout_keep(seed, offset, bh, np.arange(n), n, p)
    for causal in (False, True):
        o, _ = fwd(q, k, v, 1.0, causal, p, seed, offset, bh)
        for i in range(n):
            vis = i + 1 if causal else n
            want = z[i, :vis].sum() / (vis * (1 - float(np.float32(p))))
            assert np.max(np.abs(o[i] - want)) <= 1e-12, (causal, i)


FWD_PINS = [pin_p_zero, pin_lse_undropped, pin_expectation, pin_counts]
KEEP_PINS = [pin_keep_elementwise, pin_keep_rate, pin_streams_independent]


@pytest.mark.parametrize("pin", FWD_PINS, ids=lambda p: p.__name__)
def test_forward_pin(pin):
    pin(attention_dropout_head)


@pytest.mark.parametrize("pin", KEEP_PINS, ids=lambda p: p.__name__)
def test_keep_pin(pin):
    pin(dropout_keep)


def test_ref_and_rows_agree_with_head():
    """The batched and sampled-row forms are the per-head definition with
    bh = b * Hq + hq (and GQA head map hq // (Hq / Hkv))."""
    B, Hq, Hkv, N, d = 2, 4, 2, 10, 3
    q, k, v = _rand((B, Hq, N, d), 50), _rand((B, Hkv, N, d), 51), _rand((B, Hkv, N, d), 52)
    o, lse = attention_dropout_ref(q, k, v, True, 0.7, 0.25, 3, 1)
    for b in range(B):
        for h in range(Hq):
            oh, lh = attention_dropout_head(q[b, h], k[b, h // 2], v[b, h // 2], 0.7, True, 0.25, 3, 1, b * Hq + h)
            assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)
    rows = [(1, 3, 7), (0, 0, 0), (1, 2, 9), (0, 1, 4)]
    orow, lrow = attention_dropout_rows(q, k, v, True, 0.7, 0.25, 3, 1, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(orow[n] - o[b, h, i])) <= 1e-14 and abs(lrow[n] - lse[b, h, i]) <= 1e-14


# ---- pins of the backward ------------------------------------------------------

def _loss(q, k, v, do, scale, causal, p, seed, offset, bh):
    o, _ = attention_dropout_head(q, k, v, scale, causal, p, seed, offset, bh)
    return float(np.sum(do * o))


def pin_bwd_finite_differences(bwd):
    """Central differences of L = sum(dO * O) through the dropout forward; the
    mask depends only on (seed, offset, bh, i, j), not on Q, K or V."""
    h = 1e-6
    for n, d, causal, scale, p, seed in [(5, 3, False, 0.7, 0.3, 1), (6, 2, True, -0.45, 0.5, 2)]:
        q, k, v, do = (_rand((n, d), seed * 10 + i) for i in range(4))
        got = bwd(q, k, v, do, scale, causal, p, seed, 3, 4)
        for x, g in zip((q, k, v), got):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss(q, k, v, do, scale, causal, p, seed, 3, 4)
                x[idx] = keep - h
                lm = _loss(q, k, v, do, scale, causal, p, seed, 3, 4)
                x[idx] = keep
                num[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(num - g)) <= 1e-6 * (1 + np.max(np.abs(num))), (n, causal)


def pin_bwd_torch_autograd(bwd):
    """torch fp64 autograd of softmax(masked scores) * Z / (1 - p) @ V."""
    for n, d, causal, scale, p, seed in [(12, 5, True, 0.35, 0.2, 4), (9, 4, False, -0.8, 0.6, 5)]:
        q, k, v, do = (_rand((n, d), seed * 10 + i) for i in range(4))
        z = torch.tensor(dropout_keep(seed, 1, 2, np.arange(n), n, p).astype(np.float64))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        o = (torch.softmax(s, dim=1) * z * keep_factor(p)) @ tv
        o.backward(torch.tensor(do))
        got = bwd(q, k, v, do, scale, causal, p, seed, 1, 2)
        for g, t in zip(got, (tq, tk, tv)):
            assert np.max(np.abs(g - t.grad.numpy())) <= 1e-10, (n, causal)


def pin_bwd_p_zero(bwd):
    """p = 0: the gradients of plain attention."""
    for causal in (False, True):
        q, k, v, do = (_rand((8, 3), 60 + i) for i in range(4))
        a = bwd(q, k, v, do, 0.5, causal, 0.0, 9, 0, 0)
        b = attention_backward_head(q, k, v, do, 0.5, causal)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) <= 1e-13


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_p_zero]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(attention_dropout_backward_head)


def test_backward_gqa_group_sums():
    B, Hq, Hkv, N, d = 1, 4, 2, 7, 3
    q, do = _rand((B, Hq, N, d), 70), _rand((B, Hq, N, d), 71)
    k, v = _rand((B, Hkv, N, d), 72), _rand((B, Hkv, N, d), 73)
    dq, dk, dv = attention_dropout_backward_ref(q, k, v, do, True, 0.6, 0.3, 8, 2)
    for h in range(Hq):
        gq, gk, gv = attention_dropout_backward_head(q[0, h], k[0, h // 2], v[0, h // 2], do[0, h], 0.6,
                                                     True, 0.3, 8, 2, h)
        assert np.array_equal(dq[0, h], gq)
    want_dk = sum(attention_dropout_backward_head(q[0, h], k[0, 0], v[0, 0], do[0, h], 0.6, True, 0.3, 8, 2, h)[1]
                  for h in (0, 1))
    assert np.max(np.abs(dk[0, 0] - want_dk)) <= 1e-13


# ---- planted mistakes ------------------------------------------------------------

def _keep_mutant(inverted=False, halves_swapped=False, swapped_fields=False, ignore_bh=False,
                 plain_order=False):
    def keep(seed, offset, bh, rows, n_keys, p):
        rows = np.asarray(rows).reshape(-1)
        n_ctr = 2 * ((n_keys + 15) // 16)
        ctr = np.arange(n_ctr)[None, :]
        i = rows[:, None]
        c0, c1 = (i, ctr) if swapped_fields else (ctr, i)
        w = philox4x32_10(c0, c1, 0 if ignore_bh else bh, offset, seed & 0xFFFFFFFF, seed >> 32)
        halves = []
        for wd in np.broadcast_arrays(*w):
            lo, hi = wd & np.uint64(0xFFFF), wd >> np.uint64(16)
            halves += [hi, lo] if halves_swapped else [lo, hi]
        halves = np.stack(halves, axis=-1)
        if swapped_fields:
            halves = np.swapaxes(halves, 0, 1)
        j = np.arange(n_keys)
        if plain_order:                  # keys 8n..8n+7 on call n
            c, hf = j // 8, j % 8
        else:
            c, hf = draw_position(j)
        u = halves[:, c, hf]
        t = np.uint64(keep_threshold(p))
        return u < t if inverted else u >= t
    return keep


def _fwd_mutant(keep=dropout_keep, no_factor=False, drop_in_norm=False, transposed=False):
    def fwd(q, k, v, scale, causal, p, seed, offset, bh):
        n = q.shape[0]
        s = masked_scores(q, k, scale, causal)
        z = keep(seed, offset, bh, np.arange(n), n, p)
        if transposed:
            z = z.T
        e = s.copy()
        if drop_in_norm:
            e = np.where(z, e, -np.inf)
        pw, m, l = softmax_rows(e)
        f = 1.0 if no_factor else keep_factor(p)
        o = (pw * (1.0 if drop_in_norm else z)) @ v * (1.0 if drop_in_norm else f)
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = m + np.log(l)
        return o, lse
    return fwd


def _bwd_mutant(no_dp_mask=False, dv_from_p=False, d_from_undropped=False):
    def bwd(q, k, v, do, scale, causal, p, seed, offset, bh):
        n = q.shape[0]
        s = masked_scores(q, k, scale, causal)
        pw, _, _ = softmax_rows(s)
        zf = dropout_keep(seed, offset, bh, np.arange(n), n, p) * keep_factor(p)
        w = pw * zf
        o = (pw if d_from_undropped else w) @ v
        dv = (pw if dv_from_p else w).T @ do
        dp = (do @ v.T) * (1.0 if no_dp_mask else zf)
        ds = pw * (dp - np.sum(do * o, axis=1)[:, None])
        return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv
    return bwd


KEEP_MUTANTS = {
    "comparison inverted": _keep_mutant(inverted=True),
    "16-bit halves swapped": _keep_mutant(halves_swapped=True),
    "counter fields swapped": _keep_mutant(swapped_fields=True),
    "head unit ignored": _keep_mutant(ignore_bh=True),
    "keys in plain order on the calls": _keep_mutant(plain_order=True),
}
FWD_MUTANTS = {
    "1/(1-p) left out": _fwd_mutant(no_factor=True),
    "dropout inside the normaliser": _fwd_mutant(drop_in_norm=True),
    "mask transposed": _fwd_mutant(transposed=True),
    "comparison inverted (forward)": _fwd_mutant(keep=_keep_mutant(inverted=True)),
}
BWD_MUTANTS = {
    "dP not masked": _bwd_mutant(no_dp_mask=True),
    "dV from P instead of the dropped weights": _bwd_mutant(dv_from_p=True),
    "D from the undropped output": _bwd_mutant(d_from_undropped=True),
}


def _failures(pins, impl):
    n = 0
    for pin in pins:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            n += 1
    return n


@pytest.mark.parametrize("name", list(KEEP_MUTANTS))
def test_keep_mistakes_are_caught(name):
    assert _failures(KEEP_PINS, KEEP_MUTANTS[name]) >= 1, name


@pytest.mark.parametrize("name", list(FWD_MUTANTS))
def test_forward_mistakes_are_caught(name):
    assert _failures(FWD_PINS, FWD_MUTANTS[name]) >= 1, name


@pytest.mark.parametrize("name", list(BWD_MUTANTS))
def test_backward_mistakes_are_caught(name):
    assert _failures(BWD_PINS, BWD_MUTANTS[name]) >= 1, name


def test_unplanted_copies_pass():
    for pin in KEEP_PINS:
        pin(_keep_mutant())
    for pin in FWD_PINS:
        pin(_fwd_mutant())
    for pin in BWD_PINS:
        pin(_bwd_mutant())
