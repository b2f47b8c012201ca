"""The allocation-free split-KV entry point (partials in the library's fixed
per-device scratch array) against the split-KV entry point with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller
problem, each compared bit for bit with fa_fwd_splitkv and within the bf16
tolerances of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_04_amd.workloads import Workload, as_f64_numpy, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _launch_both(fa, w, splits):
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    stream = torch.cuda.current_stream().cuda_stream
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr())
    o_na = torch.full_like(qd, float("nan"))
    l_na = torch.full((w.B, w.Hq, w.N), float("nan"), dtype=torch.float32, device="cuda")
    _say(f"noalloc {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} splits={splits}")
    rc = fa.fa_fwd_splitkv_noalloc(*args, o_na.data_ptr(), l_na.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
                                   int(w.causal), w.scale, splits, stream)
    assert rc == fa.FA_OK, fa.fa_status_string(rc)
    need = fa.fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.N, w.d, splits)
    assert 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws = torch.empty_like(qd)
    l_ws = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd_splitkv(*args, o_ws.data_ptr(), l_ws.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
                           int(w.causal), w.scale, splits, ws.data_ptr(), need, stream)
    assert rc == fa.FA_OK, fa.fa_status_string(rc)
    torch.cuda.synchronize()
    return (q, k, v), (o_na, l_na), (o_ws, l_ws)


def test_noalloc_matches_workspace_entry_point_twice():
    from io_aware_tiled_04_amd import fa
    cases = [
        (Workload("noalloc-large", 1, 8, 2, 3000, 128, True, "bf16", 95), 4),
        # second call smaller than the first: the scratch still holds the
        # first call's partials beyond this problem's extent
        (Workload("noalloc-small", 2, 3, 3, 333, 64, False, "bf16", 96), 3),
    ]
    for w, splits in cases:
        (q, k, v), (o_na, l_na), (o_ws, l_ws) = _launch_both(fa, w, splits)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), w.name
        o_ref, lse_ref = oracle.attention_ref(*(as_f64_numpy(t) for t in (q, k, v)), w.causal, w.scale)
        err = np.abs(as_f64_numpy(o_na) - o_ref)
        lerr = np.abs(as_f64_numpy(l_na) - lse_ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3, (w.name, err.max(), lerr.max())
        _say(f"{w.name}: bitwise equal to fa_fwd_splitkv; max|dO|={err.max():.3e} max|dLSE|={lerr.max():.3e}")


def test_noalloc_rejects_oversized_problem_on_device():
    """A problem whose partials exceed the scratch array is rejected (and
    nothing is launched) also on a GPU machine."""
    from io_aware_tiled_04_amd import fa
    P = 0x1000
    rc = fa.fa_fwd_splitkv_noalloc(P, P, P, P, P, 1, 4, 4, 16384, 128, 1, 0.125, 4,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_SCRATCH
