"""Elements past the end of an input are never used.

Every tile copy of the kernels reads whole tiles: the last tile of a head
reaches past row N, into the next head or, for the last head, past the end of
the tensor.  Those rows must come back as zeros (the buffer descriptor's range
check) or be masked, never enter a result.  Each case builds every input
inside a larger buffer whose tail (what lies after the tensor) is filled once
with NaN and once with zeros, and requires bit-identical, finite outputs.
"""
import pytest
import torch

from io_aware_tiled_04_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

SLACK_ROWS = 512        # more than any tile reaches past the end


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _fa():
    from io_aware_tiled_04_amd import fa
    return fa


def _embed(t, fill):
    """t (on the GPU) copied into the front of a buffer with SLACK_ROWS rows
    of `fill` after it."""
    buf = torch.full((t.numel() + SLACK_ROWS * t.shape[-1],), fill, dtype=t.dtype, device="cuda")
    view = buf[:t.numel()].view(t.shape)
    view.copy_(t)
    return view


def _both(fn, *tensors):
    outs = []
    for fill in (float("nan"), 0.0):
        args = [_embed(t, fill) for t in tensors]
        r = fn(*args)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in r if isinstance(x, torch.Tensor)])
    for a, b in zip(*outs):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


CASES = [
    Workload("d128-causal", 1, 2, 2, 1000, 128, True, "bf16", 301),
    Workload("d128-noncausal", 1, 2, 1, 300, 128, False, "bf16", 302),
    Workload("d64-causal", 2, 2, 1, 333, 64, True, "bf16", 303),
    Workload("d64-noncausal", 1, 3, 3, 200, 64, False, "bf16", 304),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_forward_ignores_rows_past_the_end(w):
    fa = _fa()
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    _say(f"past-end fwd {w.name}")
    _both(lambda q, k, v: fa.fwd(q, k, v, causal=w.causal), q, k, v)
    _say(f"past-end fwd_splitkv {w.name}")
    _both(lambda q, k, v: fa.fwd_splitkv(q, k, v, 3, causal=w.causal), q, k, v)
    _say(f"past-end fwd_dropout {w.name}")
    _both(lambda q, k, v: fa.fwd_dropout(q, k, v, 0.2, 7, 0, causal=w.causal)[:2], q, k, v)
    _say(f"past-end fwd_kvouter {w.name}")
    _both(lambda q, k, v: fa.fwd_kvouter(q, k, v, causal=w.causal), q, k, v)


def test_forward_f32_ignores_rows_past_the_end():
    fa = _fa()
    w = Workload("f32", 1, 2, 1, 77, 64, True, "f32", 305)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    _say("past-end fwd f32")
    _both(lambda q, k, v: fa.fwd(q, k, v, causal=True), q, k, v)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_ignores_rows_past_the_end(w):
    fa = _fa()
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    o, lse = fa.fwd(q, k, v, causal=w.causal)
    g = torch.Generator().manual_seed(w.seed + 1000)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to("cuda")
    torch.cuda.synchronize()
    _say(f"past-end bwd {w.name}")
    _both(lambda q, k, v, o, lse, dout: fa.bwd(q, k, v, o, lse, dout, causal=w.causal),
          q, k, v, o, lse, dout)
