"""Thin Python binding of the C ABI in include/fa.h (ctypes).

Only argument marshalling lives here: every step of the forward pass runs in
the HIP kernels of ``libfa.so``.  There is no fallback: if the library is
missing or cannot be loaded, importing this module raises.

The ``fa_*`` functions have the C names and arguments (integer device
pointers, sizes, stream handle).  ``fwd``, ``fwd_splitkv``, ``fwd_dropout``
and ``bwd`` are the torch-facing conveniences: they check the tensors,
allocate the outputs (and any workspace) on the inputs' device and launch on
torch's current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEADS = -3
FA_ERR_HEADDIM = -4
FA_ERR_ARG = -5
FA_ERR_HIP = -6
FA_ERR_WORKSPACE = -7
FA_ERR_SCRATCH = -8
FA_ERR_ALIGN = -9

# Bytes of the fixed device scratch array of fa_fwd_splitkv_noalloc.
FA_NOALLOC_SCRATCH_BYTES = 64 << 20

# Names declared in include/fa.h, in order.
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv",
           "fa_fwd_splitkv_noalloc", "fa_fwd_dropout", "fa_fwd_kvouter_workspace_size", "fa_fwd_kvouter", "fa_bwd_workspace_size",
           "fa_bwd", "fa_bwd_dropout", "fa_status_string")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m io_aware_tiled_04_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    fwd_args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_void_p]
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = fwd_args
        fn.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = fwd_args[:-1] + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = fwd_args[:-1] + [ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_dropout.argtypes = fwd_args[:-1] + [ctypes.c_float, ctypes.c_ulonglong, ctypes.c_uint,
                                                   ctypes.c_void_p]
    lib.fa_fwd_dropout.restype = ctypes.c_int
    lib.fa_fwd_kvouter.argtypes = fwd_args[:-1] + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_fwd_kvouter.restype = ctypes.c_int
    lib.fa_fwd_kvouter_workspace_size.argtypes = [ctypes.c_int] * 4
    lib.fa_fwd_kvouter_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int] * 5
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_dropout.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_float, ctypes.c_ulonglong, ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t,
         ctypes.c_void_p]
    lib.fa_bwd_dropout.restype = ctypes.c_int
    lib.fa_bwd_workspace_size.argtypes = [ctypes.c_int] * 3
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"fa status {status}: {fa_status_string(status)}")


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream) -> int:
    """Raw call of the C entry point; pointers and stream are integers."""
    return _lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale), stream)


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, stream) -> int:
    """Raw call of the fp32 C entry point; pointers and stream are integers."""
    return _lib.fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale), stream)


def fa_fwd_splitkv_workspace_size(B, Hq, N, d, num_splits) -> int:
    """Bytes of workspace the split-KV entry point needs (0 for invalid sizes)."""
    return int(_lib.fa_fwd_splitkv_workspace_size(B, Hq, N, d, num_splits))


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, num_splits, workspace,
                   workspace_bytes, stream) -> int:
    """Raw call of the split-KV C entry point; pointers and stream are integers."""
    return _lib.fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale),
                               int(num_splits), workspace, int(workspace_bytes), stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, num_splits, stream) -> int:
    """Raw call of the allocation-free split-KV C entry point (partials in the
    library's fixed per-device scratch array); pointers and stream are
    integers."""
    return _lib.fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale),
                                       int(num_splits), stream)


def fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, p_drop, seed, offset,
                   stream) -> int:
    """Raw call of the dropout C entry point; pointers and stream are integers."""
    return _lib.fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale),
                               float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF,
                               int(offset) & 0xFFFFFFFF, stream)


def fa_fwd_kvouter_workspace_size(B, Hq, N, d) -> int:
    """Bytes of workspace the K/V-outer entry point needs (0 for invalid sizes)."""
    return int(_lib.fa_fwd_kvouter_workspace_size(B, Hq, N, d))


def fa_fwd_kvouter(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, workspace, workspace_bytes,
                   stream) -> int:
    """Raw call of the K/V-outer C entry point; pointers and stream are integers."""
    return _lib.fa_fwd_kvouter(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(scale), workspace,
                               int(workspace_bytes), stream)


def fa_bwd_workspace_size(B, Hq, N) -> int:
    """Bytes of workspace the backward entry point needs (0 for invalid sizes)."""
    return int(_lib.fa_bwd_workspace_size(B, Hq, N))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, workspace,
           workspace_bytes, stream) -> int:
    """Raw call of the backward C entry point; pointers and stream are integers."""
    return _lib.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, int(causal),
                       float(scale), workspace, int(workspace_bytes), stream)


def fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, p_drop, seed,
                   offset, workspace, workspace_bytes, stream) -> int:
    """Raw call of the dropout backward C entry point; pointers and stream are integers."""
    return _lib.fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, int(causal),
                               float(scale), float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF,
                               int(offset) & 0xFFFFFFFF, workspace, int(workspace_bytes), stream)


def _check(t, name, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU device {device}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, d]")


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse_out=None,
        stream=None):
    """Attention forward: returns (O, LSE).

    q [B,Hq,N,d], k/v [B,Hkv,N,d]: contiguous bf16 (or fp32) device tensors.
    O has q's dtype and shape; LSE is fp32 [B,Hq,N].  ``scale`` defaults to
    1/sqrt(d).  ``out`` and ``lse_out``, when given, must have exactly those
    shapes (the kernel writes B*Hq*N*d and B*Hq*N elements); every shape is
    checked before anything is launched.  Launches on ``stream`` (a torch
    stream) or torch's current stream, without synchronising.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D [B, H, N, d] torch.Tensor")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N and d")
    if out is not None and (not isinstance(out, torch.Tensor) or tuple(out.shape) != tuple(q.shape)):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}")
    if lse_out is not None and (not isinstance(lse_out, torch.Tensor) or tuple(lse_out.shape) != (B, Hq, N)):
        raise ValueError(f"lse_out must have shape {(B, Hq, N)}")
    dev = q.device
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    _check(o, "out", dtype, dev)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev:
        raise ValueError("lse_out must be a contiguous fp32 tensor on q's device")
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    fn = fa_fwd if dtype == torch.bfloat16 else fa_fwd_f32
    rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            B, Hq, Hkv, N, d, causal, scale, s)
    if rc != FA_OK:
        raise FaError(rc)
    return o, lse


def fwd_splitkv(q, k, v, num_splits: int, causal: bool = False, scale: float | None = None,
                workspace=None, stream=None):
    """Split-KV attention forward on bf16 tensors: returns (O, LSE), the same
    result as ``fwd`` up to float rounding order.

    ``workspace`` is an optional uint8 device tensor of at least
    ``fa_fwd_splitkv_workspace_size(...)`` bytes; one is allocated when it is
    None.  Launches on ``stream`` or torch's current stream.
    """
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fwd_splitkv_workspace_size(B, Hq, N, d, num_splits)
    if need == 0:
        raise ValueError("invalid sizes or num_splits for the split-KV forward")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    if workspace.data_ptr() % 16 != 0:
        raise ValueError("workspace must start at a 16-byte aligned address")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, causal, scale, num_splits, workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), s)
    if rc != FA_OK:
        raise FaError(rc)
    return o, lse


def fwd_dropout(q, k, v, p_drop: float, seed: int, offset: int = 0, causal: bool = False,
                scale: float | None = None, stream=None):
    """Attention forward with dropout on the weights, on bf16 tensors:
    returns (O, LSE, (seed, offset)).  The last item is the generator state
    that regenerates the same keep mask (the entry point draws it from
    Philox4x32-10 at that seed and offset).  LSE is that of the weights
    before dropout.  Launches on ``stream`` or torch's current stream."""
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    rc = fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, causal, scale, p_drop, seed, offset, s)
    if rc != FA_OK:
        raise FaError(rc)
    return o, lse, (int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF)


def fwd_kvouter(q, k, v, causal: bool = False, scale: float | None = None, workspace=None, stream=None):
    """The forward in the K/V-outer loop order on bf16 tensors: returns
    (O, LSE), fa_fwd's result up to float rounding order.  ``workspace``: an
    optional uint8 device tensor of at least fa_fwd_kvouter_workspace_size
    bytes (allocated when None)."""
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fwd_kvouter_workspace_size(B, Hq, N, d)
    if need == 0:
        raise ValueError("invalid sizes for the K/V-outer forward")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    rc = fa_fwd_kvouter(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                        causal, scale, workspace.data_ptr(), workspace.numel() * workspace.element_size(), s)
    if rc != FA_OK:
        raise FaError(rc)
    return o, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, workspace=None,
        stream=None, dropout=None):
    """Gradients (dQ, dK, dV) of a bf16 forward pass from its saved o and lse
    and the upstream gradient ``dout``; allocates the outputs (and the
    workspace when it is None) on q's device and launches on ``stream`` or
    torch's current stream.  ``dropout`` = (p_drop, (seed, offset)) for a
    forward run by ``fwd_dropout`` (its o, lse and returned state)."""
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, n, torch.bfloat16, dev)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N and d")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be a contiguous fp32 [B, Hq, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_bwd_workspace_size(B, Hq, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    wsz = workspace.numel() * workspace.element_size()
    if dropout is None:
        rc = fa_bwd(*ptrs, B, Hq, Hkv, N, d, causal, scale, workspace.data_ptr(), wsz, s)
    else:
        p_drop, (seed, offset) = dropout
        rc = fa_bwd_dropout(*ptrs, B, Hq, Hkv, N, d, causal, scale, p_drop, seed, offset,
                            workspace.data_ptr(), wsz, s)
    if rc != FA_OK:
        raise FaError(rc)
    return dq, dk, dv
