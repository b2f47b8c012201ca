"""Pins of the backward oracle (oracle/backward.py) to things other than itself.

Each pin takes an implementation of the per-head gradient
``impl(q, k, v, do, scale, causal) -> (dq, dk, dv)``, so the same pins also
run on planted-mistake copies and must catch every one of them:

* finite differences of the forward oracle (the definition of a gradient);
* torch's fp64 CPU autograd through scaled_dot_product_attention;
* the blog's blockwise FlashAttention backward (P recomputed from the stored
  logsumexp per block pair), over every block size;
* closed forms and invariants: equal rows of V give dQ = dK = 0; the column
  sums of dV equal those of dO; a shift of every key by one vector leaves all
  three gradients unchanged; GQA gradients are the group sums of the MHA ones.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attention_head, masked_scores, softmax_rows
from oracle.backward import attention_backward_head, attention_backward_ref, backward_blocked


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _loss(q, k, v, do, scale, causal):
    o, _ = attention_head(q, k, v, scale, causal)
    return float(np.sum(do * o))


def pin_finite_differences(impl):
    """Central differences of L = sum(dO * O(Q, K, V)) through the forward
    oracle, on tiny heads, causal and not, with positive and negative scale."""
    h = 1e-6
    for n, d, causal, scale, seed in [(5, 3, False, 0.7, 1), (6, 2, True, -0.45, 2), (4, 4, True, 1.3, 3)]:
        q, k, v, do = (_rand((n, d), seed * 10 + i) for i in range(4))
        dq, dk, dv = impl(q, k, v, do, scale, causal)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss(q, k, v, do, scale, causal)
                x[idx] = keep - h
                lm = _loss(q, k, v, do, scale, causal)
                x[idx] = keep
                num[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(num - g)) <= 1e-6 * (1 + np.max(np.abs(num))), (n, d, causal)


def pin_torch_autograd(impl):
    """torch fp64 CPU autograd of the math attention path (a library routine,
    independent of the oracle)."""
    for n, d, causal, scale, seed in [(17, 8, True, 0.35, 4), (9, 5, False, -0.8, 5)]:
        q, k, v, do = (_rand((n, d), seed * 10 + i) for i in range(4))
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
        o.backward(torch.tensor(do, dtype=torch.float64))
        dq, dk, dv = impl(q, k, v, do, scale, causal)
        for g, t in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.max(np.abs(g - t.grad.numpy())) <= 1e-10, (n, causal)


def pin_blockwise(impl):
    """The blog's blockwise backward (P recomputed from the stored LSE for
    each block pair) equals the one-shot gradient, for every block size."""
    n, d = 7, 3
    for causal, scale, seed in [(True, 0.9, 6), (False, -1.1, 7)]:
        q, k, v, do = (_rand((n, d), seed * 10 + i, 1.5) for i in range(4))
        ref = impl(q, k, v, do, scale, causal)
        for bq in (1, 2, 3, 7):
            for bk in (1, 3, 4, 7):
                got = backward_blocked(q, k, v, do, scale, causal, bq, bk)
                for a, b in zip(ref, got):
                    assert np.max(np.abs(a - b)) <= 1e-12, (bq, bk, causal)


def pin_equal_values(impl):
    """Every row of V equal to c: O = c on every row whatever P is, so the
    scores get no gradient (dQ = dK = 0); dV = P^T dO sums dO over queries,
    so sum_j dV_j = sum_i dO_i."""
    n, d = 6, 3
    for causal in (False, True):
        q, k, do = (_rand((n, d), 20 + i) for i in range(3))
        v = np.tile(_rand((1, d), 30), (n, 1))
        dq, dk, dv = impl(q, k, v, do, 0.8, causal)
        assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12
        assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12


def pin_column_sums(impl):
    """Rows of P sum to one, so for any V the column sums of dV equal those of
    dO (dV = P^T dO)."""
    n, d = 8, 4
    for causal in (False, True):
        q, k, v, do = (_rand((n, d), 40 + i) for i in range(4))
        _, _, dv = impl(q, k, v, do, 0.6, causal)
        assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12


def pin_key_shift(impl):
    """K <- K + 1 w^T adds scale * q_i . w to every score of row i, which the
    softmax cancels: O, P and hence all three gradients are unchanged (dQ
    because the rows of dS sum to zero)."""
    n, d = 6, 3
    for causal in (False, True):
        q, k, v, do = (_rand((n, d), 50 + i) for i in range(4))
        w = _rand((1, d), 59)
        a = impl(q, k, v, do, 0.7, causal)
        b = impl(q, k + w, v, do, 0.7, causal)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) <= 1e-10


PINS = [pin_finite_differences, pin_torch_autograd, pin_blockwise, pin_equal_values,
        pin_column_sums, pin_key_shift]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(attention_backward_head)


def test_rows_of_ds_sum_to_zero():
    """sum_j dS_ij = sum_j P_ij dP_ij - D_i = D_i - D_i = 0 (the property the
    key-shift pin relies on), checked directly."""
    for causal in (False, True):
        q, k, v, do = (_rand((9, 4), 70 + i) for i in range(4))
        _, _, _, ds = attention_backward_head(q, k, v, do, 0.5, causal, return_ds=True)
        assert np.max(np.abs(ds.sum(axis=1))) <= 1e-12


def test_gqa_gradients_are_group_sums():
    """Hkv < Hq: the K/V gradients of a head group are the sums of the MHA
    gradients of the group's query heads on the repeated K/V."""
    rng = np.random.default_rng(80)
    B, Hq, Hkv, N, d = 1, 4, 2, 7, 3
    q, do = rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hq, N, d))
    k, v = rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    dq, dk, dv = attention_backward_ref(q, k, v, do, True, 0.6)
    ke, ve = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = attention_backward_ref(q, ke, ve, do, True, 0.6)
    assert np.array_equal(dq, dq2)
    assert np.allclose(dk, dk2.reshape(B, Hkv, 2, N, d).sum(axis=2), atol=1e-13, rtol=0)
    assert np.allclose(dv, dv2.reshape(B, Hkv, 2, N, d).sum(axis=2), atol=1e-13, rtol=0)


# ---- planted mistakes: each must fail at least one pin ----------------------

def _mutant(drop_d=False, no_scale=False, transposed_ds=False, dv_from_ds=False, mask="causal",
            d_from_v=False, dk_uses_k=False):
    def impl(q, k, v, do, scale, causal):
        s = masked_scores(q, k, scale, causal and mask != "none")
        if causal and mask == "strict":
            n = s.shape[0]
            s = np.where(np.eye(n, dtype=bool), -np.inf, s)
            s[0, 0] = scale * q[0] @ k[0]
        p, _, _ = softmax_rows(s)
        o = p @ v
        dv = p.T @ do if not dv_from_ds else None
        dp = do @ v.T
        dsum = np.sum(do * (v if d_from_v else o), axis=1)
        ds = p * (dp - (0.0 if drop_d else dsum[:, None]))
        if transposed_ds:
            ds = ds.T
        f = 1.0 if no_scale else float(scale)
        dq = f * (ds @ k)
        dk = f * (ds.T @ (k if dk_uses_k else q))
        if dv_from_ds:
            dv = ds.T @ do
        return dq, dk, dv
    return impl


MUTANTS = {
    "D term dropped": _mutant(drop_d=True),
    "scale left out of dQ, dK": _mutant(no_scale=True),
    "dS transposed": _mutant(transposed_ds=True),
    "dV from dS instead of P": _mutant(dv_from_ds=True),
    "mask ignored": _mutant(mask="none"),
    "diagonal masked": _mutant(mask="strict"),
    "D from V instead of O": _mutant(d_from_v=True),
    "dK from K instead of Q": _mutant(dk_uses_k=True),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name):
    impl = MUTANTS[name]
    failures = 0
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures += 1
    assert failures >= 1, f"planted mistake '{name}' passed every pin"


def test_unplanted_copy_passes_every_pin():
    impl = _mutant()
    for pin in PINS:
        pin(impl)
