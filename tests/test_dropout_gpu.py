"""GPU parity of the dropout forward (fa_fwd_dropout) against the fp64 oracle.

* The keep mask is compared bit for bit: with Q = 0 every weight is exactly
  1 (row max 0, exp2(0) = 1), and with V[j] = 2^(j // d) e_(j % d) each output
  element, times (visible keys) (1 - p), is an integer code whose bits are the
  keep decisions of up to four keys.  The code is decoded from the bf16
  output (its rounding error stays below a quarter of one code step) and
  compared with the oracle's mask.
* Outputs on random inputs are compared with the oracle's dropout forward.
  The survivors' factor 1 / (1 - p) scales O and with it the bf16 rounding
  of O: |dO| <= 2e-2 + 2^-8 |O_ref| per element (half an ulp of bf16 is at
  most 2^-8 |O|) and mean |dO| <= 2e-3 / (1 - p).  LSE: <= 1e-3 as for
  fa_fwd, and bitwise equal to fa_fwd's (dropout does not touch the row
  statistics).
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_04_amd.workloads import CONFIGS, Workload, as_f64_numpy, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX_ABS, TOL_LSE = 2e-2, 1e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _fa():
    from io_aware_tiled_04_amd import fa
    return fa


def _factor(p):
    return 1.0 / (1.0 - float(np.float32(p)))


def _check_o(o, o_ref, p, tag):
    err = np.abs(o - o_ref)
    assert np.all(np.isfinite(o)), tag
    excess = err - 2.0 ** -8 * np.abs(o_ref)
    assert excess.max() <= TOL_MAX_ABS, (tag, excess.max())
    assert err.mean() <= 2e-3 * _factor(p), (tag, err.mean())
    return err.max(), err.mean()


# ---- the keep mask, bit for bit ---------------------------------------------------

MASK_CASES = [
    # B, Hq, Hkv, N, d, causal, p, seed, offset
    (2, 3, 3, 512, 128, False, 0.3, 0x1234567890ABCDEF, 5),
    (1, 2, 2, 512, 128, True, 0.5, 77, 0),
    (1, 4, 2, 300, 128, True, 0.1, 2**33 + 1, 9),
    (2, 2, 1, 256, 64, False, 0.25, 31337, 2**31 + 3),
    (1, 2, 2, 200, 64, True, 0.9, 5, 1),
    (1, 1, 1, 70, 128, False, 0.5, 6, 2),
    (1, 1, 1, 128, 64, True, 1e-6, 8, 0),      # t = floor(p 2^16) = 0: all kept, factor still 1/(1-p)
]


def _one_hot_codes(N, d):
    """V[j] = 2^(j // d) e_(j % d), bf16-exact; at most four levels."""
    assert N <= 4 * d
    v = torch.zeros(N, d)
    j = torch.arange(N)
    v[j, j % d] = (2.0 ** (j // d)).float()
    return v


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: f"N{c[3]}-d{c[4]}-{'c' if c[5] else 'nc'}-p{c[6]}")
def test_keep_mask_bit_exact(case):
    B, Hq, Hkv, N, d, causal, p, seed, offset = case
    _say(f"mask B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} p={p} seed={seed} offset={offset}")
    q = torch.zeros(B, Hq, N, d, dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    v = _one_hot_codes(N, d).to(torch.bfloat16).expand(B, Hkv, N, d).contiguous()
    o, lse, state = _fa().fwd_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, offset, causal=causal,
                                      scale=d ** -0.5)
    torch.cuda.synchronize()
    assert state == (seed, offset)
    o = as_f64_numpy(o)
    lse = as_f64_numpy(lse)
    levels = (N + d - 1) // d
    kept_total = vis_total = 0
    for b in range(B):
        for h in range(Hq):
            bh = b * Hq + h
            z = oracle.dropout_keep(seed, offset, bh, np.arange(N), N, p)
            vis = (np.arange(N) + 1) if causal else np.full(N, N)
            code = o[b, h] * vis[:, None] / _factor(p)
            ci = np.rint(code)
            assert np.max(np.abs(code - ci)) < 0.25, (b, h, np.max(np.abs(code - ci)))
            ci = ci.astype(np.int64)
            got = np.zeros((N, N), dtype=bool)
            for t in range(levels):
                cols = np.arange(t * d, min(N, (t + 1) * d))
                got[:, cols] = ((ci[:, cols - t * d] >> t) & 1).astype(bool)
            want = z.copy()
            if causal:
                want &= np.arange(N)[None, :] <= np.arange(N)[:, None]
            assert np.array_equal(got, want), (b, h, int(np.sum(got != want)))
            assert np.max(np.abs(lse[b, h] - np.log(vis))) <= 1e-5
            kept_total += int(want.sum())
            vis_total += int(vis.sum())
    # the decoded masks keep about 1 - p of the visible pairs
    frac = kept_total / vis_total
    assert abs(frac - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / vis_total) + 2.0 ** -16, frac


# ---- outputs against the oracle ---------------------------------------------------

SMALL = [
    (Workload("drop-c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31), 0.1),
    (Workload("drop-c4-small", 1, 2, 2, 700, 128, True, "bf16", 41, 2.0, 2.0, 1.0), 0.2),
    (Workload("drop-gqa", 1, 8, 2, 333, 128, True, "bf16", 51), 0.5),
    (Workload("drop-d128-noncausal", 2, 2, 2, 300, 128, False, "bf16", 62), 0.3),
    (Workload("drop-d64-causal", 2, 2, 1, 257, 64, True, "bf16", 61), 0.1),
    (Workload("drop-d64-noncausal", 1, 3, 3, 200, 64, False, "bf16", 63), 0.7),
    (Workload("drop-N1", 1, 2, 1, 1, 128, True, "bf16", 64), 0.5),
    (Workload("drop-N77", 2, 1, 1, 77, 64, False, "bf16", 67), 0.05),
]


@pytest.mark.parametrize("w,p", SMALL, ids=lambda x: x.name if hasattr(x, "name") else f"p{x}")
def test_dropout_parity_full_oracle(w, p):
    seed, offset = 1000 + w.seed, 3
    _say(f"{w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} p={p}")
    q, k, v = make_inputs(w)
    o, lse, _ = _fa().fwd_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, offset, causal=w.causal,
                                  scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_dropout_ref(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                                  w.causal, w.scale, p, seed, offset)
    _check_o(as_f64_numpy(o), o_ref, p, w.name)
    assert np.max(np.abs(as_f64_numpy(lse) - lse_ref)) <= TOL_LSE


def test_dropout_full_size_c3_sampled_rows():
    """c3 (B=2, H=32, N=4096, d=128, causal) at the launch the bench times:
    sampled rows against the oracle row by row; LSE bitwise equal to fa_fwd's
    on every row."""
    w = CONFIGS["c3"]
    p, seed, offset = 0.1, 0xC3C3C3C3DEADBEEF, 11
    _say(f"c3 dropout p={p}")
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse, _ = _fa().fwd_dropout(qd, kd, vd, p, seed, offset, causal=True, scale=w.scale)
    o0, lse0 = _fa().fwd(qd, kd, vd, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse0)
    rng = np.random.default_rng(5)
    rows = [(0, 0, 0), (1, 31, 4095), (0, 5, 255), (1, 17, 256), (0, 30, 2047)]
    rows += [(int(rng.integers(0, 2)), int(rng.integers(0, 32)), int(rng.integers(0, 4096))) for _ in range(11)]
    o_ref, lse_ref = oracle.attention_dropout_rows(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v), True,
                                                   w.scale, p, seed, offset, rows)
    on = as_f64_numpy(o)
    ln = as_f64_numpy(lse)
    got = np.stack([on[b, h, i] for b, h, i in rows])
    _check_o(got, o_ref, p, "c3 rows")
    assert np.max(np.abs(np.array([ln[b, h, i] for b, h, i in rows]) - lse_ref)) <= TOL_LSE


def test_p_zero_is_fa_fwd_and_state_reproduces():
    w = CONFIGS["c2"].with_(N=512)
    _say("p=0 and reproducibility")
    q, k, v = (t.cuda() for t in make_inputs(w))
    fa = _fa()
    o0, l0 = fa.fwd(q, k, v, causal=False, scale=w.scale)
    oz, lz, _ = fa.fwd_dropout(q, k, v, 0.0, 123, 4, causal=False, scale=w.scale)
    a1, la, st = fa.fwd_dropout(q, k, v, 0.25, 2**40 + 3, 4, causal=False, scale=w.scale)
    a2, lb, _ = fa.fwd_dropout(q, k, v, 0.25, *st, causal=False, scale=w.scale)
    a3, _, _ = fa.fwd_dropout(q, k, v, 0.25, 2**40 + 3, 5, causal=False, scale=w.scale)
    a4, _, _ = fa.fwd_dropout(q, k, v, 0.25, 3, 4, causal=False, scale=w.scale)   # high seed word differs
    torch.cuda.synchronize()
    assert torch.equal(o0, oz) and torch.equal(l0, lz)
    assert torch.equal(a1, a2) and torch.equal(la, lb) and torch.equal(la, l0)
    assert not torch.equal(a1, a3) and not torch.equal(a1, a4)


def test_dropout_rejects_bad_probability_on_device():
    fa = _fa()
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    for p in (-0.1, 1.0, float("nan")):
        with pytest.raises(fa.FaError):
            fa.fwd_dropout(q, q, q, p, 1, 0)
