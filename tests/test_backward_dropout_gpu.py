"""GPU parity of the dropout backward (fa_bwd_dropout) against the fp64 oracle.

The GPU runs fa_fwd_dropout and feeds its O and LSE, with the same generator
state, to fa_bwd_dropout, as a training step would; the oracle differentiates
the dropout forward of the same bf16 inputs.

* Random inputs: the backward's bar (max |d| <= 2e-2 and mean |d| <= 2e-3,
  relative to max |reference| of each gradient, floor 1e-4).
* Keep bits: on random inputs one wrong bit moves a gradient by about 1/N of
  its scale, below that bar, so three constructions make every bit count.
  With Q = 0 or K = 0 every weight is 1 / (visible keys), and with V and dO
  rows equal to e_0 every dP is 1:
    dQ: K = codes (row j = 2^(j // d) e_(j % d)) gives
        dQ_i[c] = scale/vis_i * sum_t (Z_i,td+c f - D_i) 2^t;
    dK: Q = codes gives dK_j[c] = scale/N * sum_t (Z_td+c,j f - D) 2^t
        (non-causal);
    dV: dO = codes gives dV_j[c] = f/N * sum_t Z_td+c,j 2^t (non-causal),
        decoded bit for bit.
  A flipped bit moves its element by at least scale f / vis (f = 1/(1-p)),
  while the rounding of P, dS and the bf16 output stays below a tenth of
  that, so the element tolerance 0.25 scale f / vis separates the two.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_04_amd.workloads import CONFIGS, Workload, as_f64_numpy, make_grad, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 2e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _fa():
    from io_aware_tiled_04_amd import fa
    return fa


def _factor(p):
    return 1.0 / (1.0 - float(np.float32(p)))


def _gpu(q, k, v, do, causal, scale, p, seed, offset):
    fa = _fa()
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    o, lse, state = fa.fwd_dropout(qd, kd, vd, p, seed, offset, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, dropout=(p, state))
    torch.cuda.synchronize()
    return as_f64_numpy(dq), as_f64_numpy(dk), as_f64_numpy(dv)


def _check(name, got, ref):
    for tag, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), (name, tag)
        scale = max(float(np.max(np.abs(r))), 1e-4)
        err = np.abs(g - r)
        assert err.max() <= TOL_MAX * scale, (name, tag, err.max(), scale)
        assert err.mean() <= TOL_MEAN * scale, (name, tag, err.mean(), scale)


CASES = [
    (Workload("bwdd-d128-causal", 1, 2, 2, 256, 128, True, "bf16", 181), 0.1),
    (Workload("bwdd-d128-noncausal-ragged", 1, 2, 2, 300, 128, False, "bf16", 182), 0.3),
    (Workload("bwdd-d64-causal-ragged", 2, 2, 1, 333, 64, True, "bf16", 183), 0.5),
    (Workload("bwdd-d64-noncausal", 1, 3, 3, 200, 64, False, "bf16", 184), 0.2),
    (Workload("bwdd-gqa-causal", 1, 8, 2, 257, 128, True, "bf16", 185), 0.1),
    (Workload("bwdd-N1", 1, 2, 1, 1, 128, True, "bf16", 187), 0.5),
    (Workload("bwdd-N77", 2, 1, 1, 77, 64, True, "bf16", 188), 0.05),
]


@pytest.mark.parametrize("w,p", CASES, ids=lambda x: x.name if hasattr(x, "name") else f"p{x}")
def test_dropout_backward_parity_full_oracle(w, p):
    seed, offset = 7000 + w.seed, 2
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say(f"bwd-dropout {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} p={p}")
    got = _gpu(q, k, v, do, w.causal, w.scale, p, seed, offset)
    ref = oracle.attention_dropout_backward_ref(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                                as_f64_numpy(do), w.causal, w.scale, p, seed, offset)
    _check(w.name, got, ref)


def _codes(N, d):
    assert N <= 4 * d
    x = torch.zeros(N, d)
    j = torch.arange(N)
    x[j, j % d] = (2.0 ** (j // d)).float()
    return x


def _e0(N, d):
    x = torch.zeros(N, d)
    x[:, 0] = 1.0
    return x


def _bf(x, B, H):
    return x.to(torch.bfloat16).expand(B, H, *x.shape).contiguous()


@pytest.mark.parametrize("N,d,causal,p", [(256, 64, True, 0.3), (200, 128, False, 0.5), (512, 128, True, 0.1)])
def test_dq_keep_bits(N, d, causal, p):
    B, Hq, Hkv, seed, offset = 1, 2, 1, 0xABCDEF0123, 4
    scale = d ** -0.5
    _say(f"bwd-dropout dQ bits N={N} d={d} causal={causal} p={p}")
    q = torch.zeros(B, Hq, N, d, dtype=torch.bfloat16)
    k, v, do = _bf(_codes(N, d), B, Hkv), _bf(_e0(N, d), B, Hkv), _bf(_e0(N, d), B, Hq)
    dq = _gpu(q, k, v, do, causal, scale, p, seed, offset)[0]
    ref = oracle.attention_dropout_backward_ref(*(as_f64_numpy(t) for t in (q, k, v, do)), causal, scale, p,
                                                seed, offset)[0]
    vis = (np.arange(N) + 1) if causal else np.full(N, N)
    tol = 0.25 * scale * _factor(p) / vis
    err = np.abs(dq - ref).max(axis=3)           # [B, Hq, N]
    assert np.all(err <= tol[None, None, :]), float(np.max(err / tol[None, None, :]))


@pytest.mark.parametrize("N,d,p", [(256, 64, 0.25), (300, 128, 0.5)])
def test_dk_keep_bits(N, d, p):
    B, Hq, Hkv, seed, offset = 1, 2, 1, 99, 0
    scale = d ** -0.5
    _say(f"bwd-dropout dK bits N={N} d={d} p={p}")
    k = torch.zeros(B, Hkv, N, d, dtype=torch.bfloat16)
    q, v, do = _bf(_codes(N, d), B, Hq), _bf(_e0(N, d), B, Hkv), _bf(_e0(N, d), B, Hq)
    dk = _gpu(q, k, v, do, False, scale, p, seed, offset)[1]
    ref = oracle.attention_dropout_backward_ref(*(as_f64_numpy(t) for t in (q, k, v, do)), False, scale, p,
                                                seed, offset)[1]
    tol = 0.25 * scale * _factor(p) / N
    assert np.max(np.abs(dk - ref)) <= tol, float(np.max(np.abs(dk - ref)) / tol)


@pytest.mark.parametrize("N,d,p", [(256, 64, 0.3), (512, 128, 0.5), (300, 128, 0.1)])
def test_dv_keep_bits_decoded(N, d, p):
    """dV_j[c] * N / f is the code sum_t Z[td + c, j] 2^t: compare the decoded
    bits with the oracle's mask, query by key, for both query heads."""
    B, Hq, Hkv, seed, offset = 1, 2, 1, 2**40 + 17, 6
    scale = d ** -0.5
    _say(f"bwd-dropout dV bits N={N} d={d} p={p}")
    q = torch.zeros(B, Hq, N, d, dtype=torch.bfloat16)
    k = torch.randn(B, Hkv, N, d, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    v = _bf(_e0(N, d), B, Hkv)
    fa = _fa()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse, state = fa.fwd_dropout(qd, kd, vd, p, seed, offset, causal=False, scale=scale)
    got = {}
    for h in range(Hq):
        # dO = codes on query head h only, so dV shows that head's mask
        do = torch.zeros(B, Hq, N, d)
        do[0, h] = _codes(N, d)
        dv = fa.bwd(qd, kd, vd, o, lse, do.to(torch.bfloat16).cuda(), causal=False, scale=scale,
                    dropout=(p, state))[2]
        torch.cuda.synchronize()
        got[h] = as_f64_numpy(dv)[0, 0]
    levels = (N + d - 1) // d
    for h in range(Hq):
        code = got[h] * N / _factor(p)               # [keys, d]
        ci = np.rint(code)
        assert np.max(np.abs(code - ci)) < 0.25, np.max(np.abs(code - ci))
        ci = ci.astype(np.int64)
        zq = np.zeros((N, N), dtype=bool)            # [query, key]
        for t in range(levels):
            rows = np.arange(t * d, min(N, (t + 1) * d))
            zq[rows, :] = ((ci[:, rows - t * d] >> t) & 1).T.astype(bool)
        want = oracle.dropout_keep(seed, offset, h, np.arange(N), N, p)
        assert np.array_equal(zq, want), (h, int(np.sum(zq != want)))


def test_dropout_backward_full_size_c3_two_heads():
    w = CONFIGS["c3"]
    p, seed, offset = 0.1, 0xC3C3, 8
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say("bwd-dropout c3 full size")
    dq, dk, dv = _gpu(q, k, v, do, True, w.scale, p, seed, offset)
    q64, k64, v64, do64 = (as_f64_numpy(t) for t in (q, k, v, do))
    for b, h in [(0, 0), (1, 31)]:
        ref = oracle.attention_dropout_backward_head(q64[b, h], k64[b, h], v64[b, h], do64[b, h], w.scale, True,
                                                     p, seed, offset, b * w.Hq + h)
        _check(f"c3 ({b},{h})", (dq[b, h], dk[b, h], dv[b, h]), ref)


def test_p_zero_is_fa_bwd_and_deterministic():
    w = Workload("bwdd-p0", 1, 4, 2, 300, 128, True, "bf16", 190)
    q, k, v = (t.cuda() for t in make_inputs(w))
    do = make_grad(w).cuda()
    _say("bwd-dropout p=0 and determinism")
    fa = _fa()
    o, lse = fa.fwd(q, k, v, causal=True, scale=w.scale)
    a = fa.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    b = fa.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale, dropout=(0.0, (5, 1)))
    od, lsed, st = fa.fwd_dropout(q, k, v, 0.4, 5, 1, causal=True, scale=w.scale)
    c1 = fa.bwd(q, k, v, od, lsed, do, causal=True, scale=w.scale, dropout=(0.4, st))
    c2 = fa.bwd(q, k, v, od, lsed, do, causal=True, scale=w.scale, dropout=(0.4, st))
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(c1, c2):
        assert torch.equal(x, y)
