"""Python binding of libffpa_attn (large-head-dimension fused attention on MI355X).

The entry points ``ffpa_attn_fwd``, ``ffpa_attn_bwd`` and the workspace queries
have the names and argument order of the C ABI in ``include/ffpa_attn.h`` and
only marshal arguments (device pointers as integers, sizes, the stream
handle). ``attention`` and ``attention_backward`` are conveniences that take
torch tensors, allocate outputs and workspace with torch and pass the current
HIP stream; every step of the computation runs in the library's kernels.

There is no fallback: if the shared library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "load", "FFPAError", "ffpa_attn_fwd", "ffpa_attn_fwd_noalloc", "ffpa_attn_bwd",
    "ffpa_attn_fwd_dropout", "ffpa_attn_bwd_dropout", "ffpa_attn_fwd_variant",
    "ffpa_attn_fwd_variant_workspace_size", "ffpa_attn_fwd_tune", "ffpa_attn_tune_reset", "tune_forward",
    "ffpa_attn_fwd_fp8", "ffpa_attn_fwd_fp8_workspace_size", "attention_fp8",
    "ffpa_attn_fwd_workspace_size",
    "ffpa_attn_bwd_workspace_size", "ffpa_attn_bwd_workspace_size_stored",
    "ffpa_attn_bwd_workspace_size_min", "ffpa_last_error",
    "ffpa_version", "attention",
    "attention_backward", "F16", "BF16", "ACC_F32", "ACC_F16", "LIB_PATH", "EXPORTED",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libffpa_attn.so")

F16, BF16 = 0, 1
ACC_F32, ACC_F16 = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
_STATUS = {1: "FFPA_ERR_INVALID_ARG", 2: "FFPA_ERR_UNSUPPORTED", 3: "FFPA_ERR_WORKSPACE",
           4: "FFPA_ERR_HIP"}

# Symbols declared in include/ffpa_attn.h.
EXPORTED = ("ffpa_attn_fwd", "ffpa_attn_fwd_workspace_size", "ffpa_attn_fwd_noalloc", "ffpa_attn_bwd",
            "ffpa_attn_bwd_workspace_size", "ffpa_attn_bwd_workspace_size_stored",
            "ffpa_attn_bwd_workspace_size_min", "ffpa_attn_fwd_dropout", "ffpa_attn_bwd_dropout", "ffpa_attn_fwd_variant",
            "ffpa_attn_fwd_variant_workspace_size", "ffpa_attn_fwd_tune", "ffpa_attn_tune_reset",
            "ffpa_attn_fwd_fp8", "ffpa_attn_fwd_fp8_workspace_size", "ffpa_last_error", "ffpa_version")

_lib: Optional[ctypes.CDLL] = None


class FFPAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library once (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FFPAError(-1, f"{path} is missing: build it with "
                            "`python -m head_dim_attention_flash_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.ffpa_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, vp, sz, vp]
    lib.ffpa_attn_fwd.restype = i
    lib.ffpa_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, vp]
    lib.ffpa_attn_fwd_noalloc.restype = i
    lib.ffpa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i,
                                  i, i, vp, sz, vp]
    lib.ffpa_attn_bwd.restype = i
    u64 = ctypes.c_uint64
    lib.ffpa_attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, f, u64,
                                          vp, sz, vp]
    lib.ffpa_attn_fwd_dropout.restype = i
    lib.ffpa_attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp,
                                          i, i, i, f, u64, vp, sz, vp]
    lib.ffpa_attn_bwd_dropout.restype = i
    lib.ffpa_attn_fwd_variant.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, i, vp, sz, vp]
    lib.ffpa_attn_fwd_variant.restype = i
    lib.ffpa_attn_fwd_variant_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.ffpa_attn_fwd_variant_workspace_size.restype = sz
    lib.ffpa_attn_fwd_tune.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, i, vp, sz, i,
                                       ctypes.POINTER(i), ctypes.POINTER(f), vp]
    lib.ffpa_attn_fwd_tune.restype = i
    lib.ffpa_attn_tune_reset.argtypes = []
    lib.ffpa_attn_tune_reset.restype = None
    lib.ffpa_attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.ffpa_attn_fwd_fp8.restype = i
    lib.ffpa_attn_fwd_fp8_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.ffpa_attn_fwd_fp8_workspace_size.restype = sz
    lib.ffpa_attn_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.ffpa_attn_fwd_workspace_size.restype = sz
    lib.ffpa_attn_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.ffpa_attn_bwd_workspace_size.restype = sz
    lib.ffpa_attn_bwd_workspace_size_stored.argtypes = [i, i, i, i, i, i, i]
    lib.ffpa_attn_bwd_workspace_size_stored.restype = sz
    lib.ffpa_attn_bwd_workspace_size_min.argtypes = [i, i, i, i, i, i, i]
    lib.ffpa_attn_bwd_workspace_size_min.restype = sz
    lib.ffpa_last_error.argtypes = []
    lib.ffpa_last_error.restype = ctypes.c_char_p
    lib.ffpa_version.argtypes = []
    lib.ffpa_version.restype = i
    _lib = lib
    return lib


def ffpa_last_error() -> str:
    return load().ffpa_last_error().decode()


def ffpa_version() -> int:
    return load().ffpa_version()


def _check(status: int) -> None:
    if status != OK:
        raise FFPAError(status, ffpa_last_error())


def ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype) -> int:
    return load().ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype)


def ffpa_attn_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype) -> int:
    return load().ffpa_attn_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype)


def ffpa_attn_bwd_workspace_size_stored(B, Hq, Hkv, Nq, Nkv, D, dtype) -> int:
    return load().ffpa_attn_bwd_workspace_size_stored(B, Hq, Hkv, Nq, Nkv, D, dtype)


def ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dtype) -> int:
    return load().ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dtype)


def ffpa_attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                  accum_dtype, dtype, workspace, workspace_bytes, stream) -> int:
    """Raw C call: pointers are integers (0 = NULL); returns the status code."""
    return load().ffpa_attn_fwd(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale, causal,
                                mask or None, mask_rows, accum_dtype, dtype, workspace or None,
                                workspace_bytes, stream or None)


def ffpa_attn_fwd_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                          accum_dtype, dtype, stream) -> int:
    """Raw C call of the forward that allocates nothing (no workspace arguments)."""
    return load().ffpa_attn_fwd_noalloc(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale,
                                        causal, mask or None, mask_rows, accum_dtype, dtype,
                                        stream or None)


def ffpa_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask,
                  mask_rows, accum_dtype, dtype, workspace, workspace_bytes, stream) -> int:
    """Raw C call: pointers are integers (0 = NULL); returns the status code."""
    return load().ffpa_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale,
                                causal, mask or None, mask_rows, accum_dtype, dtype,
                                workspace or None, workspace_bytes, stream or None)


def ffpa_attn_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                          accum_dtype, dtype, dropout_p, seed, workspace, workspace_bytes,
                          stream) -> int:
    """Raw C call of the forward with dropout on the probabilities."""
    return load().ffpa_attn_fwd_dropout(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale,
                                        causal, mask or None, mask_rows, accum_dtype, dtype,
                                        dropout_p, seed, workspace or None, workspace_bytes,
                                        stream or None)


def ffpa_attn_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, causal,
                          mask, mask_rows, accum_dtype, dtype, dropout_p, seed, workspace,
                          workspace_bytes, stream) -> int:
    """Raw C call of the backward of the forward with dropout."""
    return load().ffpa_attn_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D,
                                        scale, causal, mask or None, mask_rows, accum_dtype, dtype,
                                        dropout_p, seed, workspace or None, workspace_bytes,
                                        stream or None)


def ffpa_attn_fwd_variant(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                          accum_dtype, dtype, variant, workspace, workspace_bytes, stream) -> int:
    """Raw C call of the forward as a given variant (0 = default)."""
    return load().ffpa_attn_fwd_variant(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale, causal,
                                        mask or None, mask_rows, accum_dtype, dtype, variant,
                                        workspace or None, workspace_bytes, stream or None)


def ffpa_attn_fwd_variant_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype, causal, variant) -> int:
    return load().ffpa_attn_fwd_variant_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype, causal, variant)


def ffpa_attn_fwd_tune(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                       accum_dtype, dtype, workspace, workspace_bytes, level, stream):
    """Raw C call of the tuner; returns (status, chosen variant, [ms of variants 1..3])."""
    chosen = ctypes.c_int(0)
    ms = (ctypes.c_float * 3)(-1.0, -1.0, -1.0)
    st = load().ffpa_attn_fwd_tune(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale, causal,
                                   mask or None, mask_rows, accum_dtype, dtype, workspace or None,
                                   workspace_bytes, level, ctypes.byref(chosen), ms, stream or None)
    return st, chosen.value, list(ms)


def ffpa_attn_tune_reset() -> None:
    load().ffpa_attn_tune_reset()


def ffpa_attn_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype, workspace,
                      workspace_bytes, stream) -> int:
    """Raw C call of the fp8 forward."""
    return load().ffpa_attn_fwd_fp8(q, k, v, o, lse or None, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype,
                                    workspace or None, workspace_bytes, stream or None)


def ffpa_attn_fwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nkv, D) -> int:
    return load().ffpa_attn_fwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nkv, D)


def _seed(seed) -> int:
    seed = int(seed)
    if not 0 <= seed < 1 << 64:
        raise ValueError("seed must be an unsigned 64-bit integer")
    return seed


# ---------------------------------------------------------------------------
# torch conveniences (torch supplies device memory and the stream only)
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float16 or bfloat16")


def _accum_code(accum: str) -> int:
    if accum in ("f32", "fp32", "float32"):
        return ACC_F32
    if accum in ("f16", "fp16", "float16"):
        return ACC_F16
    raise ValueError("accum must be 'f32' or 'f16'")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Nkv, D] matching q")
    for t in (q, k, v):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("tensors must be contiguous device tensors")
        if t.dtype != q.dtype:
            raise ValueError("q, k, v must share a dtype")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    return B, Hq, Hkv, Nq, Nkv, D


def _check_tensor(t, name, shape, dtype, device):
    """Host-side check of a tensor whose pointer goes to the kernels: they read
    or write it as a dense row-major block of exactly `shape` in `dtype`."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (an expanded or strided view is not)")


def _mask_args(mask, q, Nq, Nkv):
    if mask is None:
        return 0, 0
    if mask.dtype != q.dtype or not mask.is_contiguous() or not mask.is_cuda or \
            mask.device != q.device:
        raise ValueError("mask must be a contiguous tensor in q's dtype on q's device")
    rows = mask.numel() // Nkv if Nkv else 0
    if mask.numel() != rows * Nkv or rows not in (1, Nq):
        raise ValueError("mask must have Nkv columns and 1 or Nq rows ([1,1,1,Nkv] or [1,1,Nq,Nkv])")
    return mask.data_ptr(), rows


def attention(q, k, v, *, causal: bool = False, mask=None, scale: Optional[float] = None,
              accum: str = "f32", return_lse: bool = False, out=None, lse_out=None,
              workspace=None, dropout_p: float = 0.0, seed: int = 0):
    """O = softmax(scale q k^T + mask) v on the current HIP stream (see include/ffpa_attn.h).

    dropout_p > 0 drops attention probabilities with the counter-based keep
    mask of ffpa_attn_fwd_dropout (seed: unsigned 64-bit); the backward needs
    the same dropout_p and seed."""
    import torch

    B, Hq, Hkv, Nq, Nkv, D = _dims(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        o = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.shape, q.dtype, q.device)
        o = out
    lse = None
    if lse_out is not None:
        _check_tensor(lse_out, "lse_out", (B, Hq, Nq), torch.float32, q.device)
        lse = lse_out
    elif return_lse:
        lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    mptr, mrows = _mask_args(mask, q, Nq, Nkv)
    dt = _dtype_code(q)
    ws_bytes = ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt)
    if workspace is not None and ws_bytes:
        if workspace.numel() * workspace.element_size() < ws_bytes:
            raise FFPAError(ERR_WORKSPACE, "workspace smaller than ffpa_attn_fwd_workspace_size()")
        if not workspace.is_contiguous() or workspace.device != q.device:
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws = workspace
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else 0,
            B, Hq, Hkv, Nq, Nkv, D, scale, int(causal), mptr, mrows, _accum_code(accum), dt)
    tail = (ws.data_ptr() if ws is not None else 0, ws_bytes, stream)
    if dropout_p:
        _check(ffpa_attn_fwd_dropout(*args, float(dropout_p), _seed(seed), *tail))
    else:
        _check(ffpa_attn_fwd(*args, *tail))
    return (o, lse) if return_lse else o


def tune_forward(q, k, v, *, causal: bool = False, mask=None, scale: Optional[float] = None,
                 accum: str = "f32", level: int = 2):
    """Tune the forward of this problem (ffpa_attn_fwd_tune) on scratch outputs;
    later ``attention`` calls of the same problem run the chosen variant.
    Returns (chosen variant, {variant: ms per call})."""
    import torch

    B, Hq, Hkv, Nq, Nkv, D = _dims(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device)
    mptr, mrows = _mask_args(mask, q, Nq, Nkv)
    dt = _dtype_code(q)
    # room for every variant (the largest need is the transposed copy of V)
    ws_bytes = max(ffpa_attn_fwd_variant_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dt, int(causal), var)
                   for var in range(4))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st, chosen, ms = ffpa_attn_fwd_tune(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        B, Hq, Hkv, Nq, Nkv, D, scale, int(causal), mptr, mrows,
                                        _accum_code(accum), dt, ws.data_ptr(), ws_bytes, int(level), stream)
    _check(st)
    return chosen, {i + 1: t for i, t in enumerate(ms) if t >= 0}


def attention_fp8(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                  return_lse: bool = False, out=None, workspace=None):
    """The fp8 forward (ffpa_attn_fwd_fp8) on the current HIP stream: 16-bit q, k,
    v in, quantised per head to e4m3 inside the call; output in q's dtype."""
    import torch

    B, Hq, Hkv, Nq, Nkv, D = _dims(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        o = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q.shape, q.dtype, q.device)
        o = out
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=q.device) if return_lse else None
    ws_bytes = ffpa_attn_fwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nkv, D)
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < ws_bytes or not workspace.is_contiguous() or \
                workspace.device != q.device:
            raise ValueError("workspace must be a contiguous tensor on q's device of "
                             "ffpa_attn_fwd_fp8_workspace_size() bytes")
        ws = workspace
    else:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(ffpa_attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr() if lse is not None else 0, B, Hq, Hkv, Nq, Nkv, D, scale,
                             int(causal), _dtype_code(q), ws.data_ptr(), ws_bytes, stream))
    return (o, lse) if return_lse else o


def attention_backward(dout, q, k, v, o, lse, *, causal: bool = False, mask=None,
                       scale: Optional[float] = None, store_ds: Optional[bool] = None,
                       workspace_bytes: Optional[int] = None, dropout_p: float = 0.0,
                       seed: int = 0):
    """(dq, dk, dv) of attention on the current HIP stream; o, lse from ``attention``.

    By default the call gets ffpa_attn_bwd_workspace_size bytes (for one query
    row: the decode backward's, see include/ffpa_attn.h). store_ds=True
    gives it ffpa_attn_bwd_workspace_size_stored bytes whatever Nq: the dK/dV
    pass keeps dS for the dQ pass, over chunks of kv heads whose dS fits a
    bounded buffer. store_ds=False gives it the minimum
    (ffpa_attn_bwd_workspace_size_min): dQ then recomputes S and dP.
    workspace_bytes overrides either size (at least the minimum; the library
    takes the stored-dS path when it holds K^T and one kv head's dS).
    dropout_p and seed: those of the forward (ffpa_attn_bwd_dropout)."""
    import torch

    B, Hq, Hkv, Nq, Nkv, D = _dims(q, k, v)
    _check_tensor(dout, "dout", q.shape, q.dtype, q.device)
    _check_tensor(o, "o", q.shape, q.dtype, q.device)
    _check_tensor(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    mptr, mrows = _mask_args(mask, q, Nq, Nkv)
    dt = _dtype_code(q)
    if workspace_bytes is None:
        size = {None: ffpa_attn_bwd_workspace_size, True: ffpa_attn_bwd_workspace_size_stored,
                False: ffpa_attn_bwd_workspace_size_min}[store_ds]
        workspace_bytes = size(B, Hq, Hkv, Nq, Nkv, D, dt)
    ws = torch.empty(max(workspace_bytes, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, scale, int(causal),
            mptr, mrows, ACC_F32, dt)
    tail = (ws.data_ptr(), workspace_bytes, stream)
    if dropout_p:
        _check(ffpa_attn_bwd_dropout(*args, float(dropout_p), _seed(seed), *tail))
    else:
        _check(ffpa_attn_bwd(*args, *tail))
    return dq, dk, dv
