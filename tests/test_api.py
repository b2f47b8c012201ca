"""The C ABI without a GPU: the library loads, exports every entry point that
include/fa.h declares, and rejects every invalid argument before any HIP call
(so these calls are safe on a machine with no device)."""
import ctypes
import importlib
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    assert _declared() == ["fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv_workspace_size",
                           "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_dropout", "fa_fwd_kvouter_workspace_size",
                           "fa_fwd_kvouter", "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_dropout",
                           "fa_status_string"]


def test_library_exports_every_declared_symbol():
    from io_aware_tiled_04_amd import fa
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert tuple(_declared()) == fa.EXPORTS


def test_status_codes_match_header():
    from io_aware_tiled_04_amd import fa
    text = open(HEADER).read()
    for name, val in re.findall(r"(FA_\w+)\s*=\s*(-?\d+)", text):
        assert getattr(fa, name) == int(val)
        assert fa.fa_status_string(int(val)) != "unknown status"
    assert fa.fa_status_string(12345) == "unknown status"


# Fake non-null "pointers": validation rejects these calls before any use.
P = 0x1000


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32"])
@pytest.mark.parametrize("args,expect", [
    ((0, P, P, P, P, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
    ((P, 0, P, P, P, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
    ((P, P, 0, P, P, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
    ((P, P, P, 0, P, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
    ((P, P, P, P, 0, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
    ((P, P, P, P, P, 0, 1, 1, 128, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 0, 1, 128, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 1, 0, 128, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 1, 1, 0, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 1, 1, -5, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 65536, 65536, 1, 4096, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 1, 1, (1 << 23) + 1, 64, 0, 0.125), "FA_ERR_SHAPE"),
    ((P, P, P, P, P, 1, 6, 4, 128, 64, 1, 0.125), "FA_ERR_HEADS"),
    ((P, P, P, P, P, 1, 1, 1, 128, 96, 1, 0.125), "FA_ERR_HEADDIM"),
    ((P, P, P, P, P, 1, 1, 1, 128, 256, 1, 0.125), "FA_ERR_HEADDIM"),
    ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, math.nan), "FA_ERR_ARG"),
    ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, math.inf), "FA_ERR_ARG"),
    ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, -math.inf), "FA_ERR_ARG"),
    # tensors are moved in whole 16-byte pieces; lse as 4-byte words
    ((P + 8, P, P, P, P, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
    ((P, P + 2, P, P, P, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
    ((P, P, P + 4, P, P, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
    ((P, P, P, P + 1, P, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
    ((P, P, P, P, P + 2, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
])
def test_invalid_arguments_are_rejected(fn, args, expect):
    from io_aware_tiled_04_amd import fa
    rc = getattr(fa, fn)(*args, 0)
    assert rc == getattr(fa, expect), (rc, fa.fa_status_string(rc))


def test_splitkv_rejects_the_common_invalid_arguments():
    """The split-KV entry point runs the same validation as fa_fwd first."""
    from io_aware_tiled_04_amd import fa
    W = 1 << 30
    cases = [
        ((0, P, P, P, P, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
        ((P, P, P, P, 0, 1, 1, 1, 128, 64, 0, 0.125), "FA_ERR_NULL"),
        ((P, P, P, P, P, 1, 1, 1, 0, 64, 0, 0.125), "FA_ERR_SHAPE"),
        ((P, P, P, P, P, 1, 6, 4, 128, 64, 1, 0.125), "FA_ERR_HEADS"),
        ((P, P, P, P, P, 1, 1, 1, 128, 80, 1, 0.125), "FA_ERR_HEADDIM"),
        ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, math.nan), "FA_ERR_ARG"),
        ((P, P, P, P + 8, P, 1, 1, 1, 128, 64, 1, 0.125), "FA_ERR_ALIGN"),
    ]
    for args, expect in cases:
        rc = fa.fa_fwd_splitkv(*args, 2, P, W, 0)
        assert rc == getattr(fa, expect), (args, rc)


@pytest.mark.parametrize("splits,ws,wbytes,expect", [
    (0, P, 1 << 30, "FA_ERR_ARG"),
    (-3, P, 1 << 30, "FA_ERR_ARG"),
    (257, P, 1 << 30, "FA_ERR_ARG"),
    (2, 0, 1 << 30, "FA_ERR_WORKSPACE"),
    (2, P, 0, "FA_ERR_WORKSPACE"),
    # 2 splits of [1, 4, 300, 64]: 2 * 4 * 300 * 65 * 4 bytes, one byte short
    (2, P, 2 * 4 * 300 * 65 * 4 - 1, "FA_ERR_WORKSPACE"),
    # the split kernels store float4 values: the workspace must be 16-byte aligned
    (2, P + 8, 1 << 30, "FA_ERR_WORKSPACE"),
    (2, P + 4, 1 << 30, "FA_ERR_WORKSPACE"),
])
def test_splitkv_checks_splits_and_workspace(splits, ws, wbytes, expect):
    from io_aware_tiled_04_amd import fa
    rc = fa.fa_fwd_splitkv(P, P, P, P, P, 1, 4, 2, 300, 64, 1, 0.125, splits, ws, wbytes, 0)
    assert rc == getattr(fa, expect), (rc, fa.fa_status_string(rc))


def test_splitkv_workspace_size():
    from io_aware_tiled_04_amd import fa
    assert fa.fa_fwd_splitkv_workspace_size(1, 4, 300, 64, 2) == 2 * 4 * 300 * 65 * 4
    assert fa.fa_fwd_splitkv_workspace_size(2, 32, 4096, 128, 3) == 3 * 64 * 4096 * 129 * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 128, 1) == 129 * 4
    for bad in [(0, 4, 300, 64, 2), (1, 0, 300, 64, 2), (1, 4, 0, 64, 2), (1, 4, 300, 96, 2),
                (1, 4, 300, 64, 0), (1, 4, 300, 64, 257)]:
        assert fa.fa_fwd_splitkv_workspace_size(*bad) == 0, bad


def test_dropout_rejects_invalid_arguments():
    """The dropout entry point runs fa_fwd's validation, then checks p_drop
    (0 <= p < 1, finite)."""
    from io_aware_tiled_04_amd import fa
    base = (P, P, P, P, P, 1, 2, 1, 128, 64, 1, 0.125)
    cases = [
        ((0,) + base[1:], 0.1, "FA_ERR_NULL"),
        (base[:4] + (0,) + base[5:], 0.1, "FA_ERR_NULL"),
        (base[:8] + (0,) + base[9:], 0.1, "FA_ERR_SHAPE"),
        (base[:5] + (1, 3, 2) + base[8:], 0.1, "FA_ERR_HEADS"),
        (base[:9] + (96,) + base[10:], 0.1, "FA_ERR_HEADDIM"),
        (base[:11] + (math.nan,), 0.1, "FA_ERR_ARG"),
        (base, -0.01, "FA_ERR_ARG"),
        (base, 1.0, "FA_ERR_ARG"),
        (base, 1.5, "FA_ERR_ARG"),
        (base, math.nan, "FA_ERR_ARG"),
        (base, math.inf, "FA_ERR_ARG"),
    ]
    for args, p, expect in cases:
        rc = fa.fa_fwd_dropout(*args, p, 7, 0, 0)
        assert rc == getattr(fa, expect), (args, p, rc, fa.fa_status_string(rc))


def test_kvouter_validation_and_workspace_size():
    from io_aware_tiled_04_amd import fa
    assert fa.fa_fwd_kvouter_workspace_size(2, 32, 4096, 128) == 2 * 32 * 128 * (32 * 128 + 128) * 4
    assert fa.fa_fwd_kvouter_workspace_size(1, 1, 33, 64) == 2 * (32 * 64 + 128) * 4
    for bad in [(0, 1, 64, 64), (1, 0, 64, 64), (1, 1, 0, 64), (1, 1, 64, 96)]:
        assert fa.fa_fwd_kvouter_workspace_size(*bad) == 0, bad
    need = fa.fa_fwd_kvouter_workspace_size(1, 2, 300, 64)
    base = (P, P, P, P, P, 1, 2, 1, 300, 64, 1, 0.125)
    cases = [
        ((0,) + base[1:], (P, need), "FA_ERR_NULL"),
        (base[:5] + (1, 3, 2) + base[8:], (P, need), "FA_ERR_HEADS"),
        (base[:9] + (80,) + base[10:], (P, need), "FA_ERR_HEADDIM"),
        (base[:11] + (math.inf,), (P, need), "FA_ERR_ARG"),
        (base, (0, need), "FA_ERR_WORKSPACE"),
        (base, (P + 4, need), "FA_ERR_WORKSPACE"),       # not 16-byte aligned
        (base, (P, need - 1), "FA_ERR_WORKSPACE"),
    ]
    for args, (ws, wbytes), expect in cases:
        rc = fa.fa_fwd_kvouter(*args, ws, wbytes, 0)
        assert rc == getattr(fa, expect), (args, ws, wbytes, rc, fa.fa_status_string(rc))


@pytest.mark.parametrize("ptrs,sizes,ws,expect", [
    ((0, P, P, P, P, P, P, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_NULL"),
    ((P, P, P, P, P, 0, P, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_NULL"),
    ((P, P, P, P, P, P, 0, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_NULL"),
    ((P, P, P, P, P, P, P, P, 0), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_NULL"),
    ((P, P, P, 0, P, P, P, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_NULL"),
    ((P,) * 9, (1, 2, 1, 0, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_SHAPE"),
    ((P,) * 9, (1, 3, 2, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_HEADS"),
    ((P,) * 9, (1, 2, 1, 128, 32, 1, 0.125), (P, 1 << 20), "FA_ERR_HEADDIM"),
    ((P,) * 9, (1, 2, 1, 128, 64, 1, math.inf), (P, 1 << 20), "FA_ERR_ARG"),
    ((P,) * 9, (1, 2, 1, 128, 64, 1, 0.125), (0, 1 << 20), "FA_ERR_WORKSPACE"),
    ((P,) * 9, (1, 2, 1, 128, 64, 1, 0.125), (P, 2 * 128 * 4 - 1), "FA_ERR_WORKSPACE"),
    ((P, P, P, P, P, P + 8, P, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_ALIGN"),
    ((P, P, P, P, P, P, P + 2, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_ALIGN"),
    ((P, P, P, P, P, P, P, P, P + 4), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_ALIGN"),
    ((P, P, P, P, P + 1, P, P, P, P), (1, 2, 1, 128, 64, 1, 0.125), (P, 1 << 20), "FA_ERR_ALIGN"),
])
def test_backward_rejects_invalid_arguments(ptrs, sizes, ws, expect):
    from io_aware_tiled_04_amd import fa
    rc = fa.fa_bwd(*ptrs, *sizes, *ws, 0)
    assert rc == getattr(fa, expect), (rc, fa.fa_status_string(rc))


def test_backward_dropout_rejects_invalid_arguments():
    """fa_bwd_dropout runs fa_bwd's checks, then checks p_drop."""
    from io_aware_tiled_04_amd import fa
    ptrs = (P,) * 9
    sizes = (1, 2, 1, 128, 64, 1, 0.125)
    ws = (P, 1 << 20)
    cases = [
        ((0,) + ptrs[1:], sizes, 0.1, ws, "FA_ERR_NULL"),
        (ptrs[:5] + (0,) + ptrs[6:], sizes, 0.1, ws, "FA_ERR_NULL"),
        (ptrs, (1, 3, 2, 128, 64, 1, 0.125), 0.1, ws, "FA_ERR_HEADS"),
        (ptrs, (1, 2, 1, 128, 96, 1, 0.125), 0.1, ws, "FA_ERR_HEADDIM"),
        (ptrs, sizes, 0.1, (0, 1 << 20), "FA_ERR_WORKSPACE"),
        (ptrs, sizes, 0.1, (P, 2 * 128 * 4 - 1), "FA_ERR_WORKSPACE"),
        (ptrs, sizes, -0.5, ws, "FA_ERR_ARG"),
        (ptrs, sizes, 1.0, ws, "FA_ERR_ARG"),
        (ptrs, sizes, math.nan, ws, "FA_ERR_ARG"),
    ]
    for p_, sz, pd, w_, expect in cases:
        rc = fa.fa_bwd_dropout(*p_, *sz, pd, 3, 1, *w_, 0)
        assert rc == getattr(fa, expect), (p_, sz, pd, w_, rc, fa.fa_status_string(rc))


def test_backward_workspace_size():
    from io_aware_tiled_04_amd import fa
    assert fa.fa_bwd_workspace_size(2, 32, 4096) == 2 * 32 * 4096 * 4
    assert fa.fa_bwd_workspace_size(0, 1, 1) == 0 and fa.fa_bwd_workspace_size(1, 1, -1) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No silent fallback: without libfa.so the binding refuses to load."""
    from io_aware_tiled_04_amd import fa
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "libfa.so"))
    with pytest.raises(ImportError):
        fa._load()


def test_product_path_does_not_import_the_oracle():
    """The package never imports the oracle (test infrastructure only)."""
    pkg = os.path.join(ROOT, "io_aware_tiled_04_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, flags=re.M), f
                assert "oracle/" not in src, f


def test_workloads_are_seeded_and_shaped():
    from io_aware_tiled_04_amd.workloads import CONFIGS, make_inputs
    import torch
    w = CONFIGS["c5"].with_(N=64)
    q, k, v = make_inputs(w)
    assert q.shape == (1, 32, 64, 128) and k.shape == (1, 8, 64, 128)
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    q2, _, _ = make_inputs(w)
    assert torch.equal(q, q2)
    c4 = CONFIGS["c4"].with_(N=512)
    q, k, v = make_inputs(c4)
    assert 1.8 < q.float().std().item() < 2.2 and 0.9 < v.float().std().item() < 1.1
    assert CONFIGS["c1"].dtype == "f32" and make_inputs(CONFIGS["c1"])[0].dtype == torch.float32
    assert CONFIGS["c3"].nominal_flops() == 4 * 2 * 32 * 4096 ** 2 * 128 / 2


@pytest.mark.parametrize("bad", ["out", "lse_out"])
def test_fwd_rejects_wrong_output_shapes_before_any_launch(bad):
    """A caller-supplied output of the wrong shape is rejected in the binding
    before anything reaches the library (the kernel writes B*Hq*N*d outputs
    and B*Hq*N logsumexps; a smaller buffer would be written past its end).
    The check comes before the device checks, so it holds on CPU tensors."""
    import torch
    from io_aware_tiled_04_amd import fa
    q = torch.zeros(1, 4, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    kw = {"out": torch.zeros(1, 4, 63, 128, dtype=torch.bfloat16)} if bad == "out" else \
        {"lse_out": torch.zeros(1, 4, 32, dtype=torch.float32)}
    with pytest.raises(ValueError, match=bad):
        fa.fwd(q, k, k, causal=True, **kw)
    # right shapes pass the shape checks and stop at the device check instead
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(q, k, k, causal=True, out=torch.zeros_like(q))


def test_noalloc_splitkv_rejects_before_any_hip_call():
    """The allocation-free split-KV entry point runs the common validation,
    checks the split count, and rejects a problem whose partials exceed the
    fixed scratch array (FA_ERR_SCRATCH), all before any HIP call."""
    from io_aware_tiled_04_amd import fa
    cases = [
        ((0, P, P, P, P, 1, 1, 1, 128, 64, 0, 0.125), 2, "FA_ERR_NULL"),
        ((P, P, P, P, P, 1, 6, 4, 128, 64, 1, 0.125), 2, "FA_ERR_HEADS"),
        ((P, P, P, P, P, 1, 1, 1, 128, 80, 1, 0.125), 2, "FA_ERR_HEADDIM"),
        ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, math.nan), 2, "FA_ERR_ARG"),
        ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, 0.125), 0, "FA_ERR_ARG"),
        ((P, P, P, P, P, 1, 1, 1, 128, 64, 1, 0.125), 257, "FA_ERR_ARG"),
        # 4 splits of [1, 4, 16384, 128]: 4 * 4 * 16384 * 129 * 4 bytes > 64 MiB
        ((P, P, P, P, P, 1, 4, 4, 16384, 128, 1, 0.125), 4, "FA_ERR_SCRATCH"),
        # the largest problem at 1 split that fits: B*Hq*N*(d+1)*4 <= 64 MiB
        ((P, P, P, P, P, 1, 1, 1, (64 << 20) // (129 * 4) + 1, 128, 1, 0.125), 1, "FA_ERR_SCRATCH"),
    ]
    for args, splits, expect in cases:
        rc = fa.fa_fwd_splitkv_noalloc(*args, splits, 0)
        assert rc == getattr(fa, expect), (args, splits, rc, fa.fa_status_string(rc))
    assert fa.fa_fwd_splitkv_workspace_size(1, 4, 16384, 128, 4) > fa.FA_NOALLOC_SCRATCH_BYTES
