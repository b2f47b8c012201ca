"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (absolute, over every compared element):
  bf16 inputs: max |dO| <= 2e-2 and mean |dO| <= 2e-3;
  fp32 inputs: max |dO| <= 1e-5;
  all: max |dLSE| <= 1e-3.
Reduced sizes are compared element by element against the full oracle.  The
full-size configurations are compared on every element of O and LSE against
the oracle evaluated block of rows by block of rows (the same definition:
a row of O depends only on its own query row), on sampled rows, and through
closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_tiled_04_amd.workloads import CONFIGS, Workload, as_f64_numpy, make_inputs

pytestmark = pytest.mark.gpu

TOL_BF16_MAX, TOL_BF16_MEAN, TOL_F32_MAX, TOL_LSE = 2e-2, 2e-3, 1e-5, 1e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _fa():
    from io_aware_tiled_04_amd import fa
    return fa


def _run(w: Workload, q=None, k=None, v=None):
    if q is None:
        q, k, v = make_inputs(w)
    _say(f"{w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} {w.dtype}")
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    o, lse = _fa().fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return (as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v), as_f64_numpy(o),
            as_f64_numpy(lse))


def _check(w, o, lse, o_ref, lse_ref):
    err = np.abs(o - o_ref)
    lerr = np.abs(lse - lse_ref)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    if w.dtype == "f32":
        assert err.max() <= TOL_F32_MAX, (w.name, err.max())
    else:
        assert err.max() <= TOL_BF16_MAX, (w.name, err.max())
        assert err.mean() <= TOL_BF16_MEAN, (w.name, err.mean())
    assert lerr.max() <= TOL_LSE, (w.name, lerr.max())
    return err.max(), err.mean(), lerr.max()


SMALL = [
    CONFIGS["c1"],
    CONFIGS["c2"],
    # reduced versions of the causal configurations, with ragged tails
    Workload("c3-small", 1, 3, 3, 1000, 128, True, "bf16", 31),
    Workload("c4-small", 1, 2, 2, 2100, 128, True, "bf16", 41, 2.0, 2.0, 1.0),
    Workload("c5-small", 1, 8, 2, 777, 128, True, "bf16", 51),
    Workload("d64-causal-ragged", 2, 2, 1, 333, 64, True, "bf16", 61),
    Workload("d128-noncausal-ragged", 1, 2, 2, 300, 128, False, "bf16", 62),
    Workload("d64-noncausal-ragged", 1, 3, 3, 200, 64, False, "bf16", 63, 1.5, 1.5, 1.0),
    Workload("N1-causal", 1, 2, 1, 1, 128, True, "bf16", 64),
    Workload("N1-noncausal", 1, 1, 1, 1, 64, False, "bf16", 65),
    Workload("N2-causal", 1, 1, 1, 2, 64, True, "bf16", 66),
    Workload("N77-causal", 2, 1, 1, 77, 128, True, "bf16", 67),
    Workload("N129-noncausal", 1, 1, 1, 129, 64, False, "bf16", 68),
    Workload("f32-d128-causal", 1, 2, 1, 150, 128, True, "f32", 69),
    Workload("f32-d64-ragged", 2, 1, 1, 77, 64, False, "f32", 70),
    Workload("f32-N1", 1, 1, 1, 1, 64, True, "f32", 71),
    # 32 and 64 query heads: the XCD work order that takes heads four at a time
    Workload("h32-gqa-ragged", 1, 32, 8, 300, 64, True, "bf16", 72),
    Workload("h64-noncausal-ragged", 2, 32, 32, 130, 128, False, "bf16", 73),
    # Many more query tiles than compute units, one case per branch of the
    # work order (head count a multiple of 32, a multiple of 8, neither),
    # with ragged tails and GQA.
    Workload("resident-h64-gqa-ragged", 1, 64, 16, 1100, 128, True, "bf16", 74),
    Workload("resident-h72-gqa-ragged", 3, 24, 6, 1100, 128, True, "bf16", 75),
    Workload("resident-h37-d64-ragged", 1, 37, 37, 2000, 64, True, "bf16", 76),
    Workload("resident-h80-noncausal-d64", 2, 40, 40, 900, 64, False, "bf16", 77),
    Workload("resident-h36-noncausal-ragged", 1, 36, 12, 2000, 128, False, "bf16", 78),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_parity_full_oracle(w):
    q, k, v, o, lse = _run(w)
    o_ref, lse_ref = oracle.attention_ref(q, k, v, w.causal, w.scale)
    mx, mean, lmx = _check(w, o, lse, o_ref, lse_ref)
    _say(f"{w.name}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={lmx:.3e}")


def _sample_rows(w, n_random=6, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, w.N // 2, w.N - 129, w.N - 128, w.N - 2, w.N - 1]
    rows = []
    for b in range(w.B):
        for h in range(w.Hq):
            idx = set(i for i in fixed if 0 <= i < w.N)
            idx.update(int(x) for x in rng.integers(0, w.N, n_random))
            rows.extend((b, h, i) for i in sorted(idx))
    return rows


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_parity_full_size_sampled_rows(name):
    """Full configuration, launched exactly as the bench launches it; the
    oracle evaluates sampled rows of every head."""
    w = CONFIGS[name]
    q, k, v, o, lse = _run(w)
    rows = _sample_rows(w)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, w.causal, w.scale, rows)
    idx = tuple(np.array(rows).T)
    mx, mean, lmx = _check(w, o[idx], lse[idx], o_ref, lse_ref)
    _say(f"{name} sampled {len(rows)} rows: max|dO|={mx:.3e} mean|dO|={mean:.3e} "
         f"max|dLSE|={lmx:.3e}")


def _oracle_full_in_row_blocks(w, q, k, v, rows_per_block=1024, workers=16):
    """The oracle's O and LSE for every row of every head, computed block of
    query rows by block of query rows (each block against the head's full key
    set, exactly as oracle.attention_ref does for the whole head), spread
    over a thread pool with single-threaded BLAS.  This bounds host memory
    at the long configurations (one block's S and P instead of N x N)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B, Hq, N, _ = q.shape
    o_ref = np.empty(q.shape, dtype=np.float64)
    lse_ref = np.empty((B, Hq, N), dtype=np.float64)
    jobs = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, N, rows_per_block)]

    def one(job):
        b, h, r0 = job
        r1 = min(N, r0 + rows_per_block)
        hk = oracle.kv_head(h, Hq, k.shape[1])
        o_ref[b, h, r0:r1], lse_ref[b, h, r0:r1] = oracle.attention_head(
            q[b, h, r0:r1], k[b, hk], v[b, hk], w.scale, w.causal, row_index=np.arange(r0, r1))

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, jobs))
    return o_ref, lse_ref


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_parity_full_size_every_element(name):
    """Full configuration on its seeded inputs, launched exactly as the bench
    launches it: every element of O and LSE against the fp64 oracle, with the
    tolerances taken over all elements (max and mean |dO|, max |dLSE|)."""
    import time
    w = CONFIGS[name]
    q, k, v, o, lse = _run(w)
    t0 = time.perf_counter()
    o_ref, lse_ref = _oracle_full_in_row_blocks(w, q, k, v)
    mx, mean, lmx = _check(w, o, lse, o_ref, lse_ref)
    _say(f"{name} every element ({o.size} O, {lse.size} LSE; oracle {time.perf_counter() - t0:.1f} s): "
         f"max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={lmx:.3e}")


LONG = [
    # 16384 key tiles for the last rows, ragged tail, one query head
    Workload("long-causal-d128", 1, 1, 1, (1 << 20) - 3, 128, True, "bf16", 91),
    # GQA pair at d = 64, non-causal, ragged
    Workload("long-noncausal-d64-gqa", 1, 2, 1, (1 << 17) + 1, 64, False, "bf16", 92),
]


@pytest.mark.parametrize("w", LONG, ids=lambda w: w.name)
def test_long_sequences_sampled_rows(w):
    """Long sequences (far more key tiles per row than any configuration): the
    sampled rows of every head against the oracle.  The interface admits N up
    to 2^23; a causal head at that length is about 2e16 FLOPs (many seconds)
    and 2 GiB per input, so the test stops at 2^20."""
    q, k, v, o, lse = _run(w)
    rows = _sample_rows(w, n_random=4)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, w.causal, w.scale, rows)
    idx = tuple(np.array(rows).T)
    mx, mean, lmx = _check(w, o[idx], lse[idx], o_ref, lse_ref)
    _say(f"{w.name} sampled {len(rows)} rows: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={lmx:.3e}")


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_full_size_constant_scores_closed_form(name):
    """Q = 0 (exact in bf16): every allowed key has weight 1/(i+1), so
    O_i = mean(v_0..v_i) and LSE_i = ln(i+1) on every element of the full
    configuration."""
    w = CONFIGS[name]
    q, k, v = make_inputs(w)
    q = torch.zeros_like(q)
    q64, k64, v64, o, lse = _run(w, q, k, v)
    g = w.Hq // w.Hkv
    vv = np.repeat(v64, g, axis=1)
    cm = np.cumsum(vv, axis=2) / np.arange(1, w.N + 1)[None, None, :, None]
    ln = np.log(np.arange(1, w.N + 1))[None, None, :]
    _check(w, o, lse, cm, np.broadcast_to(ln, lse.shape))


def test_full_size_v_ones():
    """Rows of P sum to one: V = 1 gives O = 1 on every element of c4 (wide
    logits, long rows)."""
    w = CONFIGS["c4"]
    q, k, v = make_inputs(w)
    v = torch.ones_like(v)
    _, _, _, o, _ = _run(w, q, k, v)
    assert np.max(np.abs(o - 1.0)) <= 2.0 ** -8


def test_first_causal_row_is_v0():
    w = CONFIGS["c3"]
    q, k, v, o, lse = _run(w)
    assert np.max(np.abs(o[:, :, 0, :] - v[:, :, 0, :])) <= 2.0 ** -8 * np.max(np.abs(v[:, :, 0]))
    ref = w.scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - ref)) <= TOL_LSE


@pytest.mark.parametrize("slope", [0.5, -0.5, 2.0])
@pytest.mark.parametrize("causal", [True, False])
def test_logits_that_move_every_tile(slope, causal):
    """Scaled logits that rise (or fall) by `slope` per key.  Rising by 0.5,
    every 64-key tile's max exceeds the reference of the tiles before by
    about 46 in log2 units, so every tile moves the reference (with finite
    weights above the row-sum limit) and rescales O and l; rising by 2, the
    weights against the old reference overflow fp32 in every tile, so every
    tile takes the exact row max from S recomputed; falling, the first
    tile's reference holds and the later weights underflow to zero.  Q is
    zero but for one column of ones (exact in bf16), so the logits come from
    that column of K alone."""
    w = Workload("moving-max", 1, 2, 1, 1000, 128, causal, "bf16", 85)
    g = torch.Generator().manual_seed(85)
    q = torch.zeros(w.B, w.Hq, w.N, w.d)
    q[..., 0] = 1.0
    k = 0.1 * torch.randn(w.B, w.Hkv, w.N, w.d, generator=g)
    k[..., 0] = slope * torch.arange(w.N, dtype=torch.float32) / w.scale
    v = torch.randn(w.B, w.Hkv, w.N, w.d, generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    q64, k64, v64, o, lse = _run(w, q, k, v)
    o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, w.causal, w.scale)
    mx, mean, lmx = _check(w, o, lse, o_ref, lse_ref)
    _say(f"moving max slope={slope} causal={causal}: max|dO|={mx:.3e} mean|dO|={mean:.3e} max|dLSE|={lmx:.3e}")


def test_gqa_equals_mha_bitwise():
    """The GQA head map equals plain multi-head attention on K/V repeated per
    group, bit for bit."""
    fa = _fa()
    w = Workload("gqa", 1, 8, 2, 700, 128, True, "bf16", 81)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    _say("gqa vs mha")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k.repeat_interleave(4, dim=1).contiguous(),
                    v.repeat_interleave(4, dim=1).contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic_and_no_out_of_bounds_writes():
    """Two launches give identical bits, and nothing is written past O or LSE
    (canary padding)."""
    fa = _fa()
    w = Workload("canary", 2, 4, 2, 333, 128, True, "bf16", 82)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    pad = 4096
    outs = []
    for _ in range(2):
        ob = torch.full((q.numel() + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
        lb = torch.full((w.B * w.Hq * w.N + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
        o = ob[pad:pad + q.numel()].view(q.shape)
        lse = lb[pad:pad + w.B * w.Hq * w.N].view(w.B, w.Hq, w.N)
        _say("canary launch")
        fa.fwd(q, k, v, causal=True, out=o, lse_out=lse)
        torch.cuda.synchronize()
        assert torch.all(ob[:pad] == 7.0) and torch.all(ob[-pad:] == 7.0)
        assert torch.all(lb[:pad] == 7.0) and torch.all(lb[-pad:] == 7.0)
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_worked_example_at_kernel_shape_f32():
    """The Polish notes' worked example scaled up to the fp32 kernel's shape:
    256 keys, half with score 0 and value 0, half with score ln 3 and value 1;
    weights 1:3, so every output is 384/512 = 0.75 and LSE = ln 512.  The two
    128-key halves alone give 0 and 1, whose mean 0.5 is wrong."""
    fa = _fa()
    N, d = 256, 64
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[0, 0, 128:, 0] = math.log(3.0)
    v = torch.zeros(1, 1, N, d)
    v[0, 0, 128:, :] = 1.0
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    _say("worked example f32")
    o, lse = fa.fwd(qd, kd, vd, causal=False, scale=1.0)
    # each half on its own (queries and keys have equal length in the ABI, and
    # every query is the same vector, so 128 of them stand for all)
    qh = qd[:, :, :128].contiguous()
    oa, _ = fa.fwd(qh, kd[:, :, :128].contiguous(), vd[:, :, :128].contiguous(), scale=1.0)
    ob, _ = fa.fwd(qh, kd[:, :, 128:].contiguous(), vd[:, :, 128:].contiguous(), scale=1.0)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o - 0.75)).item() <= 1e-6
    assert torch.max(torch.abs(lse - math.log(512.0))).item() <= 1e-5
    assert torch.all(oa == 0.0) and torch.max(torch.abs(ob - 1.0)).item() <= 1e-6
    assert torch.max(torch.abs(0.5 * (oa + ob) - 0.5)).item() <= 1e-6
    assert torch.min(torch.abs(0.5 * (oa + ob) - o[:, :, :128])).item() >= 0.25 - 1e-6


def test_worked_example_at_kernel_shape_bf16():
    """The same construction in bf16 (ln 3 rounds to 1.09375 in bf16, so the
    exact answer is the oracle's on the rounded inputs, about 0.7489)."""
    fa = _fa()
    N, d = 256, 128
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[0, 0, 128:, 0] = math.log(3.0)
    v = torch.zeros(1, 1, N, d)
    v[0, 0, 128:, :] = 1.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    _say("worked example bf16")
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=False, scale=1.0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(*(as_f64_numpy(t) for t in (q, k, v)), False, 1.0)
    assert abs(o_ref[0, 0, 0, 0] - 0.75) < 2e-3
    assert np.max(np.abs(as_f64_numpy(o) - o_ref)) <= 2.0 ** -8
    assert np.max(np.abs(as_f64_numpy(lse) - lse_ref)) <= 1e-4


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.7])
def test_other_scales(scale):
    """Zero and negative scales (the kernel folds the sign into Q)."""
    w = Workload("scales", 1, 2, 2, 200, 128, True, "bf16", 83)
    q, k, v = make_inputs(w)
    _say(f"scale={scale}")
    o, lse = _fa().fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(*(as_f64_numpy(t) for t in (q, k, v)), True, scale)
    _check(w, as_f64_numpy(o), as_f64_numpy(lse), o_ref, lse_ref)


def test_side_stream():
    """The launch goes to the given stream (asynchronous, no implicit sync)."""
    fa = _fa()
    w = Workload("stream", 1, 2, 2, 256, 64, True, "bf16", 84)
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    _say("side stream")
    with torch.cuda.stream(s):
        o, lse = fa.fwd(qd, kd, vd, causal=True, stream=s)
    s.synchronize()
    o_ref, lse_ref = oracle.attention_ref(*(as_f64_numpy(t) for t in (q, k, v)), True, w.scale)
    _check(w, as_f64_numpy(o), as_f64_numpy(lse), o_ref, lse_ref)


def test_concurrent_streams_and_host_threads():
    """Two different problems launched at once, from two host threads, each on
    its own stream (both at the default priority), give bit for bit the
    results of running each alone: the library keeps no state between calls."""
    import threading
    fa = _fa()
    ws = [Workload("conc-a", 2, 8, 2, 1500, 128, True, "bf16", 86),
          Workload("conc-b", 1, 16, 16, 700, 64, False, "bf16", 87)]
    ins = [tuple(t.cuda() for t in make_inputs(w)) for w in ws]
    _say("concurrent streams: serial reference")
    alone = []
    for w, (q, k, v) in zip(ws, ins):
        alone.append(fa.fwd(q, k, v, causal=w.causal, scale=w.scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in ws]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [None] * len(ws)
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                q, k, v = ins[i]
                res = []
                for _ in range(5):
                    res.append(fa.fwd(q, k, v, causal=ws[i].causal, scale=ws[i].scale, stream=streams[i]))
                outs[i] = res
        except Exception as e:  # pragma: no cover
            errors.append(e)

    _say("concurrent streams: two host threads")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(ws))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(ws)):
        for o, lse in outs[i]:
            assert torch.equal(o, alone[i][0]) and torch.equal(lse, alone[i][1]), ws[i].name


def test_misaligned_tensors_are_rejected_before_any_launch():
    """Views that start 2 bytes into their storage (contiguous, bf16) are
    refused with FA_ERR_ALIGN, and the output is left untouched."""
    w = Workload("align", 1, 2, 2, 128, 64, False, "bf16", 93)
    q, k, v = (t.to("cuda") for t in make_inputs(w))
    fa = _fa()
    shifted = torch.empty(q.numel() + 1, dtype=torch.bfloat16, device="cuda")[1:].view(q.shape)
    shifted.copy_(q)
    out = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 128), 7.0, dtype=torch.float32, device="cuda")
    _say("misaligned q rejected")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(shifted, k, v, scale=w.scale, out=out, lse_out=lse)
    assert e.value.status == fa.FA_ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
