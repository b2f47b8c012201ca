"""GPU parity of the backward pass (fa_bwd) against the fp64 backward oracle.

The pages fix no tolerance for gradients.  The bar is the forward's bf16 bar
applied relative to each gradient tensor's magnitude: max |d| <= 2e-2 and
mean |d| <= 2e-3, both times max(max |reference|, 1e-4) of that tensor (dQ,
dK and dV separately).  The inputs round P and dS to bf16 for the matrix products
(relative 2^-9 each) and the outputs to bf16 (2^-9), with fp32 accumulation,
so the measured errors sit well below this bar.

The GPU runs the forward first (fa_fwd) and feeds its bf16 O and fp32 LSE to
the backward, as a training step would; the oracle differentiates the exact
attention of the same bf16 inputs.
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


def _gpu_grads(w, q, k, v, do, scale=None):
    scale = w.scale if scale is None else scale
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    o, lse = _fa().fwd(qd, kd, vd, causal=w.causal, scale=scale)
    dq, dk, dv = _fa().bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    return as_f64_numpy(dq), as_f64_numpy(dk), as_f64_numpy(dv)


def _check(name, got, ref):
    out = []
    for tag, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), (name, tag)
        # A gradient can vanish by cancellation (one visible key: dS = dP - D
        # = 0), where only rounding residue remains; the magnitude floor of
        # 1e-4 keeps the bar meaningful there (inputs are O(1)).
        scale = max(float(np.max(np.abs(r))), 1e-4)
        err = np.abs(g - r)
        assert err.max() <= TOL_MAX * scale, (name, tag, err.max(), scale)
        assert err.mean() <= TOL_MEAN * scale, (name, tag, err.mean(), scale)
        out.append(f"{tag} max {err.max() / scale:.2e} mean {err.mean() / scale:.2e}")
    return "; ".join(out)


CASES = [
    Workload("bwd-d128-causal", 1, 2, 2, 256, 128, True, "bf16", 81),
    Workload("bwd-d128-noncausal-ragged", 1, 2, 2, 300, 128, False, "bf16", 82),
    Workload("bwd-d64-causal-ragged", 2, 2, 1, 333, 64, True, "bf16", 83),
    Workload("bwd-d64-noncausal", 1, 3, 3, 200, 64, False, "bf16", 84, 1.5, 1.5, 1.0),
    Workload("bwd-gqa-causal", 1, 8, 2, 257, 128, True, "bf16", 85),
    Workload("bwd-wide-logits", 1, 2, 2, 520, 128, True, "bf16", 86, 2.0, 2.0, 1.0),
    Workload("bwd-N1", 1, 2, 1, 1, 128, True, "bf16", 87),
    Workload("bwd-N77", 2, 1, 1, 77, 64, True, "bf16", 88),
    Workload("bwd-c3-small", 1, 2, 2, 1000, 128, True, "bf16", 89),
    # whole dK/dV steps only (three 32-row tiles per step at d = 64, two at d = 128), and a GQA
    # group at d = 64 whose heads each end on a full step
    Workload("bwd-d64-whole-steps", 1, 2, 2, 192, 64, False, "bf16", 93),
    Workload("bwd-d128-one-step", 1, 2, 2, 64, 128, True, "bf16", 94),
    Workload("bwd-d64-gqa-whole-steps", 1, 4, 1, 288, 64, True, "bf16", 95),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_parity_full_oracle(w):
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say(f"bwd {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal}")
    got = _gpu_grads(w, q, k, v, do)
    ref = oracle.attention_backward_ref(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                        as_f64_numpy(do), w.causal, w.scale)
    _say(f"bwd {w.name}: {_check(w.name, got, ref)}")


def test_backward_full_size_c3_two_heads():
    """c3 at full size, launched as the bench launches it; the oracle checks
    two whole heads (each head's gradients depend only on that head)."""
    w = CONFIGS["c3"]
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say("bwd c3 full size")
    dq, dk, dv = _gpu_grads(w, q, k, v, do)
    q64, k64, v64, do64 = (as_f64_numpy(t) for t in (q, k, v, do))
    for b, h in [(0, 0), (1, 31)]:
        ref = oracle.attention_backward_head(q64[b, h], k64[b, h], v64[b, h], do64[b, h], w.scale, True)
        _say(f"bwd c3 head ({b},{h}): {_check('c3', (dq[b, h], dk[b, h], dv[b, h]), ref)}")


def test_backward_negative_scale():
    w = Workload("bwd-neg-scale", 1, 2, 2, 160, 64, True, "bf16", 90)
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say("bwd negative scale")
    got = _gpu_grads(w, q, k, v, do, scale=-0.2)
    ref = oracle.attention_backward_ref(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                        as_f64_numpy(do), True, -0.2)
    _say(f"bwd negative scale: {_check(w.name, got, ref)}")


def test_backward_equal_values_give_no_score_gradient():
    """Closed form on the GPU: every row of V equal gives dQ = dK = 0 (up to
    the rounding of O and of dS), whatever P is."""
    w = Workload("bwd-equal-v", 1, 2, 2, 256, 128, True, "bf16", 91)
    q, k, v = make_inputs(w)
    v = v[:, :, :1, :].expand_as(v).contiguous()
    do = make_grad(w)
    _say("bwd equal V rows")
    dq, dk, dv = _gpu_grads(w, q, k, v, do)
    ref_dv = oracle.attention_backward_ref(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                           as_f64_numpy(do), True, w.scale)[2]
    scale = np.max(np.abs(ref_dv))
    assert np.max(np.abs(dq)) <= 2e-2 * scale and np.max(np.abs(dk)) <= 2e-2 * scale
    assert np.max(np.abs(dv - ref_dv)) <= 2e-2 * scale


def test_backward_is_deterministic():
    w = Workload("bwd-det", 1, 4, 2, 300, 128, True, "bf16", 92)
    q, k, v = make_inputs(w)
    do = make_grad(w)
    _say("bwd determinism")
    a = _gpu_grads(w, q, k, v, do)
    b = _gpu_grads(w, q, k, v, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
