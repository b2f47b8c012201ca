"""Pins for the fp64 oracle, against what the pages and the mathematics fix.

Each ``pin_*`` takes an attention implementation with the oracle's signature
``impl(q, k, v, causal, scale) -> (O, LSE)`` over [B, H, N, d] arrays, so the
same pins run on the real oracle and on copies of it with a planted mistake
(``test_planted_mistakes_are_caught``): every such mistake must fail at least
one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention_ref, attention_rows, softmax_rows, masked_scores
from oracle import recurrence as rec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# --------------------------------------------------------------------------
# pins


def pin_worked_example(impl):
    """Polish notes, worked example: scores [0,0,ln3,ln3], values [0,0,1,1]
    give 6/8 = 0.75; the two blocks give 0 and 1; their mean 0.5 is wrong."""
    with open(os.path.join(GOLDEN, "worked_example_p2.json")) as f:
        g = json.load(f)
    scores = np.array([0.0 if s == "0" else math.log(3.0) for s in g["scores"]])
    vals = np.array(g["values"])
    # one query q=1 (d=1), key j = score_j, scale 1: q.k_j = score_j
    q = np.ones((1, 1, 4, 1))
    k = scores.reshape(1, 1, 4, 1)
    v = vals.reshape(1, 1, 4, 1)
    o, lse = impl(q, k, v, False, 1.0)
    assert np.all(np.abs(o[..., 0] - g["result"]) <= 1e-15), o
    assert g["result"] == g["result_fraction"][0] / g["result_fraction"][1]
    w = np.array(g["unnormalised_weight_ratios"], dtype=float)
    assert np.allclose(np.exp(scores), w, rtol=1e-15)
    assert np.all(np.abs(lse - math.log(w.sum())) <= 1e-14), lse
    # per-block results and the wrong block average
    a = g["block_split"][0]
    o1, _ = impl(q, k[:, :, :a], v[:, :, :a], False, 1.0)
    o2, _ = impl(q, k[:, :, a:], v[:, :, a:], False, 1.0)
    assert np.allclose(o1[0, 0, :, 0], g["block_results"][0], atol=1e-15)
    assert np.allclose(o2[0, 0, :, 0], g["block_results"][1], atol=1e-15)
    naive = 0.5 * (o1 + o2)
    assert np.allclose(naive, g["naive_block_average"], atol=1e-15)
    assert np.all(np.abs(naive - o) > 0.2)


def pin_v_ones(impl):
    """Rows of P sum to one over the allowed keys (Polish notes: weights are
    normalised over all allowed keys): V == 1 gives O == 1."""
    for causal in (False, True):
        for (B, H, N, d, sig) in ((1, 2, 37, 8, 1.0), (2, 1, 64, 4, 4.0)):
            q = _rand((B, H, N, d), 1, sig)
            k = _rand((B, H, N, d), 2, sig)
            v = np.ones((B, H, N, 3))
            o, _ = impl(q, k, v, causal, 1.0 / math.sqrt(d))
            assert np.max(np.abs(o - 1.0)) <= 1e-12


def pin_first_causal_row(impl):
    """The first query of a causal head sees only key 0: O_0 = v_0 exactly and
    LSE_0 = scale * q_0 . k_0."""
    B, H, N, d = 2, 3, 19, 5
    q, k, v = _rand((B, H, N, d), 3), _rand((B, H, N, d), 4), _rand((B, H, N, d), 5)
    sc = 0.37
    o, lse = impl(q, k, v, True, sc)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])
    ref = sc * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - ref)) <= 1e-13


def pin_constant_scores(impl):
    """Q == 0 makes every score 0: P is uniform over the allowed keys.
    Causal: O_i = mean(v_0..v_i), LSE_i = ln(i+1); else O_i = mean(v), ln N."""
    B, H, N, d = 1, 2, 33, 4
    q = np.zeros((B, H, N, d))
    k, v = _rand((B, H, N, d), 6), _rand((B, H, N, d), 7)
    o, lse = impl(q, k, v, True, 0.5)
    cm = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.max(np.abs(o - cm)) <= 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, N + 1))[None, None, :])) <= 1e-13
    o, lse = impl(q, k, v, False, 0.5)
    assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) <= 1e-13
    assert np.max(np.abs(lse - math.log(N))) <= 1e-13


def pin_dominant_key(impl):
    """One key whose logit beats every other by 50: the output is that key's
    value to within N*e^-50 (rescaling by the running max is exact)."""
    N, d, j = 24, 4, 7
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, j, 0] = 50.0
    v = _rand((1, 1, N, 3), 8)
    for causal in (False, True):
        o, lse = impl(q, k, v, causal, 1.0)
        rows = np.arange(N) if not causal else np.arange(j, N)
        assert np.max(np.abs(o[0, 0, rows] - v[0, 0, j])) <= N * math.exp(-50) * 10
        assert np.max(np.abs(lse[0, 0, rows] - 50.0)) <= 1e-12
        if causal:  # rows before the dominant key: plain prefix means
            cm = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
            assert np.max(np.abs(o[0, 0, :j] - cm[:j])) <= 1e-13


def pin_key_shift(impl):
    """Adding the same vector w to every key shifts every logit of row i by
    scale*q_i.w: O is unchanged and LSE_i grows by scale*q_i.w."""
    B, H, N, d = 1, 2, 29, 6
    q, k, v = _rand((B, H, N, d), 9), _rand((B, H, N, d), 10), _rand((B, H, N, d), 11)
    w = _rand((d,), 12, 3.0)
    sc = 0.41
    for causal in (False, True):
        o0, l0 = impl(q, k, v, causal, sc)
        o1, l1 = impl(q, k + w, v, causal, sc)
        assert np.max(np.abs(o1 - o0)) <= 1e-12
        assert np.max(np.abs(l1 - l0 - sc * (q @ w))) <= 1e-11


def pin_key_permutation(impl):
    """Without a mask the key order does not matter (Polish notes: a block's
    share is its weight, not its position): permuting K and V rows jointly
    leaves O and LSE unchanged."""
    B, H, N, d = 2, 1, 31, 5
    q, k, v = _rand((B, H, N, d), 13), _rand((B, H, N, d), 14), _rand((B, H, N, d), 15)
    perm = np.random.default_rng(16).permutation(N)
    o0, l0 = impl(q, k, v, False, 0.3)
    o1, l1 = impl(q, k[:, :, perm], v[:, :, perm], False, 0.3)
    assert np.max(np.abs(o1 - o0)) <= 1e-13
    assert np.max(np.abs(l1 - l0)) <= 1e-13


def pin_gqa_equals_mha(impl):
    """Grouped-query heads equal plain multi-head attention on K/V repeated
    per group (contiguous groups), bit for bit."""
    B, Hq, Hkv, N, d = 2, 6, 2, 17, 4
    q = _rand((B, Hq, N, d), 17)
    k, v = _rand((B, Hkv, N, d), 18), _rand((B, Hkv, N, d), 19)
    for causal in (False, True):
        o0, l0 = impl(q, k, v, causal, 0.5)
        o1, l1 = impl(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1),
                      causal, 0.5)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def _one_head(impl, q, k, v, causal, scale):
    o, lse = impl(q[None, None], k[None, None], v[None, None], causal, scale)
    return o[0, 0], lse[0, 0]


def pin_block_merge(impl, quick=False):
    """Two-block online merge equals the one-shot result, by brute force on
    tiny inputs, for the three page forms of the rescaled recurrence (reading
    notes' normalised O; Polish notes' u/l; the blog's exponential-domain m with
    C), at every split point; plus chains of equal blocks of every size and
    the blog's per-key recurrence."""
    Ns = (1, 2, 3, 5, 8) if quick else range(1, 9)
    seed = 100
    for N in Ns:
        for d in (1, 2, 3):
            for sig in (0.5, 3.0, 10.0):
                for causal in (False, True):
                    seed += 1
                    q, k, v = _rand((N, d), seed, sig), _rand((N, d), seed + 1000, sig), \
                        _rand((N, d), seed + 2000)
                    sc = 1.0 / math.sqrt(d)
                    o, lse = _one_head(impl, q, k, v, causal, sc)
                    tol_o = 1e-12 * max(1.0, np.max(np.abs(v)))
                    # largest |LSE| is about sig^2 * d * sc -> relative bound
                    tol_l = 1e-12 * max(1.0, np.max(np.abs(lse)))
                    forms = [rec.online_normalised, rec.online_u_over_l]
                    if sig <= 3.0:
                        forms.append(rec.blocked_exp_domain)
                    for cut in range(1, N):
                        for form in forms:
                            o2, l2 = form(q, k, v, sc, causal, [cut, N - cut])
                            assert np.max(np.abs(o2 - o)) <= tol_o, (form.__name__, N, d, sig, cut)
                            assert np.max(np.abs(l2 - lse)) <= tol_l, (form.__name__, N, d, sig, cut)
                    for bs in range(1, N + 1):
                        o2, l2 = rec.online_u_over_l(q, k, v, sc, causal, bs)
                        assert np.max(np.abs(o2 - o)) <= tol_o
                        assert np.max(np.abs(l2 - lse)) <= tol_l
                    if sig <= 3.0:
                        o2, l2 = rec.per_key_recurrence(q, k, v, sc, causal)
                        assert np.max(np.abs(o2 - o)) <= 1e-11 * max(1.0, np.max(np.abs(v)))
                        assert np.max(np.abs(l2 - lse)) <= 1e-11 * max(1.0, np.max(np.abs(lse)))


def pin_torch_sdpa(impl):
    """An independent library routine: torch's CPU float64 attention (math
    path) for O and torch.logsumexp of the masked scaled scores for LSE."""
    for (B, H, N, d, causal, sig) in ((1, 2, 70, 16, True, 1.0), (2, 1, 45, 8, False, 2.0),
                                      (1, 1, 130, 32, True, 2.0)):
        q, k, v = _rand((B, H, N, d), 30 + N, sig), _rand((B, H, N, d), 31 + N, sig), \
            _rand((B, H, N, d), 32 + N)
        sc = 1.0 / math.sqrt(d)
        o, lse = impl(q, k, v, causal, sc)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                              scale=sc)
        assert np.max(np.abs(o - to.numpy())) <= 1e-10
        ts = torch.matmul(tq, tk.transpose(-1, -2)) * sc
        if causal:
            ts = ts.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        assert np.max(np.abs(lse - torch.logsumexp(ts, dim=-1).numpy())) <= 1e-10


PINS = [pin_worked_example, pin_v_ones, pin_first_causal_row, pin_constant_scores,
        pin_dominant_key, pin_key_shift, pin_key_permutation, pin_gqa_equals_mha,
        pin_block_merge, pin_torch_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_ref)


# --------------------------------------------------------------------------
# direct checks of the oracle's building blocks


def test_rows_of_p_sum_to_one():
    """Pin (b) at the configurations' score statistics: every row of P sums to
    one to 1e-12, including wide (std 4) logits and causal rows."""
    for (N, d, sig, causal) in ((256, 64, 1.0, False), (512, 128, 2.0, True),
                                (300, 128, 1.0, True)):
        q, k = _rand((N, d), 40, sig), _rand((N, d), 41, sig)
        s = masked_scores(q, k, 1.0 / math.sqrt(d), causal)
        p, m, l = softmax_rows(s)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
        if causal:
            assert np.all(p[np.triu_indices(N, 1)] == 0.0)


def test_rows_subset_matches_full():
    """``attention_rows`` (sampled rows for the big configurations) gives the
    same rows as the full oracle."""
    B, Hq, Hkv, N, d = 1, 4, 2, 90, 16
    q = _rand((B, Hq, N, d), 50)
    k, v = _rand((B, Hkv, N, d), 51), _rand((B, Hkv, N, d), 52)
    o, lse = attention_ref(q, k, v, True, 0.25)
    rows = [(0, 3, 0), (0, 0, 89), (0, 1, 45), (0, 2, 7), (0, 3, 88)]
    o2, l2 = attention_rows(q, k, v, True, 0.25, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o2[n] - o[b, h, i])) <= 1e-13
        assert abs(l2[n] - lse[b, h, i]) <= 1e-13


def test_fully_masked_row_definition():
    """A row with no visible key (unreachable through the entry points) is
    defined as O = 0, LSE = -inf."""
    q, k, v = _rand((3, 2), 60), _rand((3, 2), 61), _rand((3, 2), 62)
    from oracle import attention_head
    o, lse = attention_head(q, k, v, 1.0, True, row_index=np.array([-1, 0, 2]))
    assert np.all(o[0] == 0.0) and lse[0] == -np.inf
    assert np.array_equal(o[1], v[0])


def test_merge_partials_equals_one_shot():
    """Merging the outputs of two disjoint key sets by their LSE weights gives
    the one-shot result (the rescale rule applied to whole partial results)."""
    N, d = 40, 8
    q, k, v = _rand((N, d), 70, 2.0), _rand((N, d), 71, 2.0), _rand((N, d), 72)
    o, lse = _one_head(attention_ref, q, k, v, False, 0.35)
    for cut in (1, 13, 39):
        o1, l1 = _one_head(attention_ref, q, k[:cut], v[:cut], False, 0.35)
        o2, l2 = _one_head(attention_ref, q, k[cut:], v[cut:], False, 0.35)
        om, lm = rec.merge_partials(o1, l1, o2, l2)
        assert np.max(np.abs(om - o)) <= 1e-13
        assert np.max(np.abs(lm - lse)) <= 1e-13


def test_blocked_without_rescale_is_exact_for_small_logits():
    """The blog's unrescaled blocked form agrees for small logits (it only
    lacks overflow protection)."""
    N, d = 20, 4
    q, k, v = _rand((N, d), 80, 0.5), _rand((N, d), 81, 0.5), _rand((N, d), 82)
    o, _ = _one_head(attention_ref, q, k, v, True, 0.5)
    for bs in (1, 3, 7, 20):
        assert np.max(np.abs(rec.blocked_no_rescale(q, k, v, 0.5, True, bs) - o)) <= 1e-13


# --------------------------------------------------------------------------
# planted mistakes: each copy of the oracle below is wrong in one plausible
# way, and at least one pin must reject it.


def _mutant(score_fn=None, mask="causal", normalise=True, lse_fn=None, head_map=None,
            use_k_as_v=False, drop_last=False, axis=1):
    def impl(q, k, v, causal, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        Nk = k.shape[2]
        o = np.empty((B, Hq, N, v.shape[3]))
        lse = np.empty((B, Hq, N))
        for b in range(B):
            for h in range(Hq):
                hk = head_map(h, Hq, Hkv) if head_map else h // (Hq // Hkv)
                kk, vv = k[b, hk], (k[b, hk] if use_k_as_v else v[b, hk])
                s = score_fn(q[b, h], kk, scale) if score_fn else scale * q[b, h] @ kk.T
                if causal:
                    rows, cols = np.arange(N)[:, None], np.arange(Nk)[None, :]
                    bad = {"causal": cols > rows, "strict": cols >= rows,
                           "upper": cols < rows, "zero": cols > rows}[mask]
                    s = np.where(bad, 0.0 if mask == "zero" else -np.inf, s)
                if drop_last:
                    s = s[:, :-1] if s.shape[1] > 1 else s
                    vv = vv[:-1] if vv.shape[0] > 1 else vv
                with np.errstate(all="ignore"):
                    m = np.max(s, axis=axis, keepdims=True)
                    e = np.exp(s - m)
                    l = e.sum(axis=axis, keepdims=True)
                    p = e / l if normalise else e
                    o[b, h] = p @ vv
                    mm, ll = (m[:, 0], l[:, 0]) if axis == 1 else (np.max(s, 1), l[0, :N])
                    lse[b, h] = lse_fn(mm, ll) if lse_fn else mm + np.log(ll)
        return o, lse
    return impl


MUTANTS = {
    "scale dropped": _mutant(score_fn=lambda q, k, s: q @ k.T),
    "scale square-rooted": _mutant(score_fn=lambda q, k, s: math.sqrt(s) * q @ k.T),
    "K and Q swapped (S transposed)": _mutant(score_fn=lambda q, k, s: s * (k @ q.T)),
    "diagonal masked": _mutant(mask="strict"),
    "mask transposed": _mutant(mask="upper"),
    "masked logit 0 instead of -inf": _mutant(mask="zero"),
    "no normalisation": _mutant(normalise=False),
    "LSE in log2": _mutant(lse_fn=lambda m, l: m + np.log2(l)),
    "LSE without the max": _mutant(lse_fn=lambda m, l: np.log(l)),
    "GQA head = hq mod Hkv": _mutant(head_map=lambda h, hq, hkv: h % hkv),
    "K used as V": _mutant(use_k_as_v=True),
    "last key dropped": _mutant(drop_last=True),
    "softmax over queries": _mutant(axis=0),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name):
    impl = MUTANTS[name]
    failures = 0
    for pin in PINS:
        try:
            if pin is pin_block_merge:
                pin(impl, quick=True)
            else:
                pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures += 1
    assert failures >= 1, f"planted mistake '{name}' passed every pin"


def test_unplanted_copy_passes_every_pin():
    """The mutant scaffold with no mistake passes, so the catches above are
    caused by the planted mistakes and not by the scaffold."""
    impl = _mutant()
    for pin in PINS:
        if pin is pin_block_merge:
            pin(impl, quick=True)
        else:
            pin(impl)
