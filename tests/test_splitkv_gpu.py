"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the fp64 oracle.

The split-KV path computes partial results over disjoint key ranges and merges
them with the rescaling rule of the reading-notes page (Methods, the two
rescaling equations), applied to whole ranges.  Its output must match the
oracle to the same tolerances as fa_fwd (bf16: max |dO| <= 2e-2 and
mean |dO| <= 2e-3; max |dLSE| <= 1e-3), for every split count, including
counts that leave some ranges empty and rows that see no key of a range.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_04_amd.workloads import CONFIGS, Workload, as_f64_numpy, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _fa():
    from io_aware_tiled_04_amd import fa
    return fa


def _check(name, o, lse, o_ref, lse_ref):
    err = np.abs(o - o_ref)
    lerr = np.abs(lse - lse_ref)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), name
    assert err.max() <= TOL_MAX, (name, err.max())
    assert err.mean() <= TOL_MEAN, (name, err.mean())
    assert lerr.max() <= TOL_LSE, (name, lerr.max())
    return err.max(), err.mean(), lerr.max()


CASES = [
    (Workload("c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31), 2),
    (Workload("c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31), 3),
    (Workload("c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31), 7),
    (Workload("c4-small", 1, 2, 2, 2100, 128, True, "bf16", 41, 2.0, 2.0, 1.0), 5),
    (Workload("c5-small", 1, 8, 2, 777, 128, True, "bf16", 51), 4),
    (Workload("d64-causal-ragged", 2, 2, 1, 333, 64, True, "bf16", 61), 3),
    (Workload("d128-noncausal-ragged", 1, 2, 2, 300, 128, False, "bf16", 62), 2),
    (Workload("d64-noncausal-ragged", 1, 3, 3, 200, 64, False, "bf16", 63, 1.5, 1.5, 1.0), 4),
    # more splits than key tiles: some ranges are empty
    (Workload("N77-causal", 2, 1, 1, 77, 128, True, "bf16", 67), 3),
    (Workload("N1-causal", 1, 2, 1, 1, 128, True, "bf16", 64), 2),
    (Workload("N300-noncausal-256splits", 1, 1, 1, 300, 64, False, "bf16", 72), 256),
    (CONFIGS["c2"], 2),
]


@pytest.mark.parametrize("w,splits", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_splitkv_parity_full_oracle(w, splits):
    q, k, v = make_inputs(w)
    _say(f"splitkv {w.name} S={splits} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal}")
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    need = _fa().fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.N, w.d, splits)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")  # contents must not matter
    o, lse = _fa().fwd_splitkv(qd, kd, vd, splits, causal=w.causal, scale=w.scale,
                               workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    q64, k64, v64 = as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v)
    o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, w.causal, w.scale)
    mx, mean, lmx = _check(w.name, as_f64_numpy(o), as_f64_numpy(lse), o_ref, lse_ref)
    _say(f"splitkv {w.name} S={splits}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={lmx:.3e}")


def test_splitkv_full_size_sampled_rows():
    """c3 at full size with 4 splits, against the oracle on sampled rows."""
    w = CONFIGS["c3"]
    q, k, v = make_inputs(w)
    _say("splitkv c3 full size S=4")
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    o, lse = _fa().fwd_splitkv(qd, kd, vd, 4, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = [(b, h, int(i)) for b in range(w.B) for h in range(w.Hq)
            for i in [0, 63, 64, 1023, 1024, 2047, 2048, 4095] + list(rng.integers(0, w.N, 3))]
    q64, k64, v64 = as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v)
    o_ref, lse_ref = oracle.attention_rows(q64, k64, v64, True, w.scale, rows)
    idx = tuple(np.array(rows).T)
    mx, mean, lmx = _check("c3-S4", as_f64_numpy(o)[idx], as_f64_numpy(lse)[idx], o_ref, lse_ref)
    _say(f"splitkv c3 S=4 sampled {len(rows)} rows: max|dO|={mx:.3e} mean|dO|={mean:.3e} "
         f"max|dLSE|={lmx:.3e}")


def test_splitkv_one_split_matches_the_direct_path_closely():
    """With one split the partial is the whole result: after the fp32 round
    trip through the workspace it must agree with fa_fwd to bf16 rounding."""
    w = Workload("c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    _say("splitkv S=1 vs fa_fwd")
    o1, l1 = _fa().fwd(q, k, v, causal=True, scale=w.scale)
    o2, l2 = _fa().fwd_splitkv(q, k, v, 1, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.allclose(o1.float(), o2.float(), atol=2 ** -8, rtol=2 ** -7)
    assert torch.allclose(l1, l2, atol=1e-5, rtol=0)


def test_splitkv_is_deterministic_and_reuses_its_workspace():
    w = Workload("c5-small", 1, 8, 2, 777, 128, True, "bf16", 51)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    _say("splitkv determinism S=3")
    need = _fa().fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.N, w.d, 3)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, l1 = _fa().fwd_splitkv(q, k, v, 3, causal=True, scale=w.scale, workspace=ws)
    o2, l2 = _fa().fwd_splitkv(q, k, v, 3, causal=True, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_rejects_a_small_workspace_without_launching():
    w = Workload("tiny", 1, 2, 2, 128, 64, False, "bf16", 9)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    need = _fa().fa_fwd_splitkv_workspace_size(1, 2, 128, 64, 2)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(_fa().FaError) as e:
        _fa().fwd_splitkv(q, k, v, 2, workspace=ws)
    assert e.value.status == _fa().FA_ERR_WORKSPACE
