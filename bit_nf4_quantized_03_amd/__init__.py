"""Python binding of the QLoRA NF4 HIP library (libqlora_nf4.so).

The functions carry the names of the C entry points in include/qlora_nf4.h
and only marshal arguments: torch supplies device memory (outputs and
workspaces are allocated with torch on the input's device) and the current
HIP stream; every step of the computation runs in the library's kernels.
Importing this package fails loudly if the library has not been built
(``python bit_nf4_quantized_03_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

__all__ = [
    "LIB_PATH", "lib", "QLORA_F32", "QLORA_BF16", "QloraError", "NF4Weight",
    "qlora_nf4_storage_bytes", "qlora_nf4_codebook", "qlora_nf4_quantize_workspace_bytes",
    "qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_workspace_bytes",
    "qlora_linear_fwd", "qlora_linear_bwd", "qlora_last_error", "EXPORTED_SYMBOLS",
    "qlora_profile_enable", "qlora_profile_read", "qlora_profile_reset",
    "qlora_weight_storage_bytes", "qlora_format_levels", "format_has_dq",
    "QLORA_FMT_NF4_DQ", "QLORA_FMT_NF4", "QLORA_FMT_FP4_DQ", "QLORA_FMT_FP4",
    "qlora_nf4_merge_workspace_bytes", "qlora_nf4_merge",
    "qlora_adamw_workspace_bytes", "qlora_adamw_step", "linear_workspace", "LINEAR_SYNC_BYTES",
    "qlora_linear_fwd_noalloc", "qlora_linear_fwd_save", "qlora_linear_bwd_saved",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora_nf4.so")

QLORA_F32 = 0
QLORA_BF16 = 1

EXPORTED_SYMBOLS = (
    "qlora_nf4_storage_bytes", "qlora_nf4_codebook", "qlora_nf4_quantize_workspace_bytes",
    "qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_workspace_bytes",
    "qlora_linear_fwd", "qlora_linear_bwd", "qlora_last_error",
    "qlora_profile_enable", "qlora_profile_read", "qlora_profile_reset",
    "qlora_weight_storage_bytes", "qlora_format_levels",
    "qlora_nf4_merge_workspace_bytes", "qlora_nf4_merge",
    "qlora_adamw_workspace_bytes", "qlora_adamw_step", "qlora_linear_fwd_noalloc",
    "qlora_linear_fwd_save", "qlora_linear_bwd_saved",
)


class QloraError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
        ("dq_scale", ctypes.c_void_p), ("dq_mean", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p), ("format", ctypes.c_int32),
    ]


class _AdamwHparams(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in ("lr", "beta1", "beta2", "eps", "weight_decay")] + \
        [("step", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python bit_nf4_quantized_03_amd/build.py`")
    # torch ships its own HIP runtime under the soname the library links
    # against (libamdhip64.so.7). Loading torch first makes the library bind
    # to that same runtime; loading the library first would put a second HIP
    # runtime in the process, which then finds no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, i32, f32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    wp = ctypes.POINTER(_Weight)
    sigs = {
        "qlora_nf4_storage_bytes": (sz, [i64, i64]),
        "qlora_nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "qlora_weight_storage_bytes": (sz, [i64, i64, ctypes.c_int]),
        "qlora_format_levels": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_float)]),
        "qlora_nf4_quantize_workspace_bytes": (sz, [i64, i64]),
        "qlora_nf4_quantize": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, wp, vp, sz, vp]),
        "qlora_nf4_dequantize": (ctypes.c_int, [wp, vp, ctypes.c_int, vp]),
        "qlora_linear_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "qlora_linear_fwd": (ctypes.c_int, [vp, i64, wp, vp, vp, i32, f32, vp, vp, sz, vp]),
        "qlora_linear_bwd": (ctypes.c_int, [vp, vp, i64, wp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "qlora_linear_fwd_noalloc": (ctypes.c_int, [vp, i64, wp, vp, vp, i32, f32, vp, vp]),
        "qlora_linear_fwd_save": (ctypes.c_int, [vp, i64, wp, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "qlora_linear_bwd_saved": (ctypes.c_int,
                                   [vp, vp, vp, i64, wp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "qlora_nf4_merge_workspace_bytes": (sz, [i64, i64, i32]),
        "qlora_nf4_merge": (ctypes.c_int, [wp, vp, vp, i32, f32, wp, vp, sz, vp]),
        "qlora_adamw_workspace_bytes": (sz, [i64, ctypes.c_int]),
        "qlora_adamw_step": (ctypes.c_int, [vp, vp, vp, vp, i64, ctypes.POINTER(_AdamwHparams), ctypes.c_int,
                                            vp, sz, vp]),
        "qlora_last_error": (ctypes.c_char_p, []),
        "qlora_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "qlora_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_int64)]),
        "qlora_profile_reset": (ctypes.c_int, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def qlora_last_error() -> str:
    return lib.qlora_last_error().decode()


def _check(fn: str, status: int):
    if status != 0:
        raise QloraError(fn, status, qlora_last_error())


def qlora_nf4_storage_bytes(rows: int, cols: int) -> int:
    return int(lib.qlora_nf4_storage_bytes(rows, cols))


def qlora_nf4_codebook():
    """The library's 16 NF4 levels as a list of Python floats (fp32 values)."""
    buf = (ctypes.c_float * 16)()
    _check("qlora_nf4_codebook", lib.qlora_nf4_codebook(buf))
    return [buf[i] for i in range(16)]


# weight formats (qlora_format): bit 0 = no double quantization, bit 1 = FP4 levels
QLORA_FMT_NF4_DQ = 0
QLORA_FMT_NF4 = 1
QLORA_FMT_FP4_DQ = 2
QLORA_FMT_FP4 = 3


def format_has_dq(fmt: int) -> bool:
    return (fmt & 1) == 0


def qlora_weight_storage_bytes(rows: int, cols: int, fmt: int) -> int:
    return int(lib.qlora_weight_storage_bytes(rows, cols, fmt))


def qlora_format_levels(fmt: int):
    """The 16 levels of weight format ``fmt`` as a list of Python floats (fp32 values)."""
    buf = (ctypes.c_float * 16)()
    _check("qlora_format_levels", lib.qlora_format_levels(fmt, buf))
    return [buf[i] for i in range(16)]


def qlora_nf4_quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib.qlora_nf4_quantize_workspace_bytes(rows, cols))


def qlora_linear_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return int(lib.qlora_linear_workspace_bytes(M, N, K, r))


QLORA_PROF_FWD_GEMM = 0
QLORA_PROF_BWD_DX = 1
QLORA_PROF_QUANTIZE = 2
QLORA_PROF_DEQUANTIZE = 3


def qlora_profile_enable(on: bool = True) -> None:
    _check("qlora_profile_enable", lib.qlora_profile_enable(1 if on else 0))


def qlora_profile_read(kind: int):
    """(total milliseconds, launches) recorded for ``kind`` since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("qlora_profile_read", lib.qlora_profile_read(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def qlora_profile_reset() -> None:
    _check("qlora_profile_reset", lib.qlora_profile_reset())


# ---------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _need_cuda(name, t, dtype=None, shape=None, device=None):
    """Check that ``t`` is a contiguous CUDA (HIP) tensor of ``dtype``, exactly
    ``shape`` and on ``device`` (each check only when given). The C ABI takes
    bare pointers, so these checks are what keeps a short or misplaced tensor
    from being read or written out of bounds on the GPU."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _need_ws(ws, device):
    """A caller-supplied workspace: a contiguous CUDA tensor on ``device``
    (its size is checked by the library)."""
    _need_cuda("ws", ws, device=device)


def _adapter(W, A, B, device):
    """Rank of the adapter (A [r, K], B [N, r], fp32) or 0 without one."""
    torch = _torch()
    if A is None and B is None:
        return 0
    if A is None or B is None:
        raise ValueError("A and B must both be given or both be None")
    _need_cuda("A", A, torch.float32, device=device)
    if A.dim() != 2 or A.shape[0] < 1:
        raise ValueError(f"A must be [r, {W.cols}] with r >= 1")
    r = A.shape[0]
    _need_cuda("A", A, shape=(r, W.cols))
    _need_cuda("B", B, torch.float32, (W.rows, r), device)
    return r


@dataclasses.dataclass
class NF4Weight:
    """4-bit weight [rows, cols] held in device tensors, in format ``fmt``
    (NF4 + DQ by default). With DQ: absmax_q, dq_scale, dq_mean; without:
    the fp32 block constants ``absmax`` (the other three are None)."""
    rows: int
    cols: int
    codes: "object"      # uint8 [ceil(n/2)]
    absmax_q: "object"   # int8 [nb], or None
    dq_scale: "object"   # float32 [nd], or None
    dq_mean: "object"    # float32 [1], or None
    absmax: "object" = None   # float32 [nb] without DQ
    fmt: int = QLORA_FMT_NF4_DQ

    @staticmethod
    def empty(rows: int, cols: int, device, fmt: int = QLORA_FMT_NF4_DQ) -> "NF4Weight":
        torch = _torch()
        n = rows * cols
        nb = -(-n // 64)
        nd = -(-nb // 256)
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=device)
        if not format_has_dq(fmt):
            return NF4Weight(rows, cols, codes, None, None, None,
                             torch.empty(nb, dtype=torch.float32, device=device), fmt)
        return NF4Weight(rows, cols, codes,
                         torch.empty(nb, dtype=torch.int8, device=device),
                         torch.empty(nd, dtype=torch.float32, device=device),
                         torch.empty(1, dtype=torch.float32, device=device), None, fmt)

    def c_struct(self) -> _Weight:
        return _Weight(self.rows, self.cols, _ptr(self.codes), _ptr(self.absmax_q),
                       _ptr(self.dq_scale), _ptr(self.dq_mean), _ptr(self.absmax), self.fmt)

    @property
    def device(self):
        return self.codes.device


def qlora_nf4_quantize(W, out: Optional[NF4Weight] = None, ws=None, fmt: Optional[int] = None) -> NF4Weight:
    """Quantize a 2-D fp32 or bf16 CUDA tensor to 4-bit codes in format ``fmt``
    (``out.fmt`` when ``out`` is given, else NF4 + DQ)."""
    torch = _torch()
    _need_cuda("W", W)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    if W.dtype == torch.float32:
        dt = QLORA_F32
    elif W.dtype == torch.bfloat16:
        dt = QLORA_BF16
    else:
        raise TypeError(f"W must be float32 or bfloat16, got {W.dtype}")
    rows, cols = W.shape
    if out is None:
        out = NF4Weight.empty(rows, cols, W.device, QLORA_FMT_NF4_DQ if fmt is None else fmt)
    elif fmt is not None and fmt != out.fmt:
        raise ValueError(f"fmt {fmt} differs from out.fmt {out.fmt}")
    if ws is None and format_has_dq(out.fmt):
        need = qlora_nf4_quantize_workspace_bytes(rows, cols)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=W.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = out.c_struct()
    _check("qlora_nf4_quantize",
           lib.qlora_nf4_quantize(_ptr(W), dt, rows, cols, ctypes.byref(st), _ptr(ws),
                                  ws_bytes, _stream_ptr(W.device)))
    return out


def qlora_nf4_dequantize(q: NF4Weight, dtype=None, out=None):
    """Dequantize to a [rows, cols] tensor of ``dtype`` (float32 or bfloat16)."""
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if dtype == torch.float32:
        dt = QLORA_F32
    elif dtype == torch.bfloat16:
        dt = QLORA_BF16
    else:
        raise TypeError(f"dtype must be float32 or bfloat16, got {dtype}")
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.device)
    else:
        _need_cuda("out", out, dtype, (q.rows, q.cols), q.device)
    st = q.c_struct()
    _check("qlora_nf4_dequantize",
           lib.qlora_nf4_dequantize(ctypes.byref(st), _ptr(out), dt, _stream_ptr(q.device)))
    return out


def qlora_nf4_merge_workspace_bytes(rows: int, cols: int, r: int) -> int:
    return int(lib.qlora_nf4_merge_workspace_bytes(rows, cols, r))


def qlora_nf4_merge(W: NF4Weight, A=None, B=None, scale: float = 0.0, out: Optional[NF4Weight] = None,
                    ws=None, fmt: Optional[int] = None) -> NF4Weight:
    """Merge s * B A into the quantized base W and quantize the result again
    into ``out`` (a new weight in format ``fmt``, default W's format)."""
    torch = _torch()
    r = _adapter(W, A, B, W.device)
    if out is None:
        out = NF4Weight.empty(W.rows, W.cols, W.device, W.fmt if fmt is None else fmt)
    need = qlora_nf4_merge_workspace_bytes(W.rows, W.cols, r)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=W.device)
    else:
        _need_ws(ws, W.device)
    sw, so = W.c_struct(), out.c_struct()
    _check("qlora_nf4_merge",
           lib.qlora_nf4_merge(ctypes.byref(sw), _ptr(A), _ptr(B), r, float(scale), ctypes.byref(so), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream_ptr(W.device)))
    return out


def qlora_adamw_workspace_bytes(n: int, state_on_host: bool) -> int:
    return int(lib.qlora_adamw_workspace_bytes(n, 1 if state_on_host else 0))


def qlora_adamw_step(param, grad, m, v, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0, ws=None) -> None:
    """One AdamW step in place on fp32 ``param`` and its state ``m``, ``v``.
    param and grad are CUDA tensors; m and v are CUDA tensors, or pinned CPU
    tensors (the state paged from host memory). ``step`` is t >= 1; the
    library forms the bias corrections from it."""
    torch = _torch()
    _need_cuda("param", param, torch.float32)
    _need_cuda("grad", grad, torch.float32, device=param.device)
    n = param.numel()
    on_host = not m.is_cuda
    for name, t in (("m", m), ("v", v)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
        if t.is_cuda == on_host or (on_host and not t.is_pinned()):
            raise ValueError("m and v must both be CUDA tensors or both pinned CPU tensors")
    if grad.numel() != n or step < 1:
        raise ValueError("grad must match param and step must be >= 1")
    if not on_host and (m.device != param.device or v.device != param.device):
        raise ValueError("m and v must be on param's device")
    hp = _AdamwHparams(lr, beta1, beta2, eps, weight_decay, int(step))
    need = qlora_adamw_workspace_bytes(n, on_host)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=param.device)
    elif need:
        _need_ws(ws, param.device)
    _check("qlora_adamw_step",
           lib.qlora_adamw_step(_ptr(param), _ptr(grad), _ptr(m), _ptr(v), n, ctypes.byref(hp),
                                1 if on_host else 0, _ptr(ws) if need else None,
                                ws.numel() * ws.element_size() if need else 0, _stream_ptr(param.device)))


# Bytes of synchronization words at the start of every linear workspace: they
# must be zero before the workspace's first use (the library leaves them zero).
LINEAR_SYNC_BYTES = 256 * 1024


def linear_workspace(M: int, N: int, K: int, r: int, device):
    """A workspace for qlora_linear_fwd / qlora_linear_bwd at these sizes,
    allocated zero-filled (its leading synchronization words must start at
    zero; every call leaves them zero again)."""
    torch = _torch()
    need = qlora_linear_workspace_bytes(M, N, K, r)
    if need == 0:
        raise ValueError(f"invalid linear sizes M={M} N={N} K={K} r={r}")
    return torch.zeros(need, dtype=torch.uint8, device=device)


def _linear_ws(M, N, K, r, device, ws):
    if ws is None:
        return linear_workspace(M, N, K, r, device)
    _need_ws(ws, device)
    return ws


def _activation(name, X, W: NF4Weight):
    """Rows M of a bf16 activation [M, W.cols] on W's device."""
    torch = _torch()
    _need_cuda(name, X, torch.bfloat16, device=W.device)
    if X.dim() != 2 or X.shape[0] < 1:
        raise ValueError(f"{name} must be 2-D [M, {W.cols}] with M >= 1")
    _need_cuda(name, X, shape=(X.shape[0], W.cols))
    return X.shape[0]


def qlora_linear_fwd(X, W: NF4Weight, A=None, B=None, scale: float = 0.0, ws=None, out=None):
    """Y = X W^T + scale (X A^T) B^T; X bf16 [M, K], A fp32 [r, K], B fp32 [N, r]."""
    torch = _torch()
    M = _activation("X", X, W)
    K, N = W.cols, W.rows
    r = _adapter(W, A, B, W.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    else:
        _need_cuda("out", out, torch.bfloat16, (M, N), W.device)
    ws = _linear_ws(M, N, K, r, X.device, ws)
    st = W.c_struct()
    _check("qlora_linear_fwd",
           lib.qlora_linear_fwd(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale),
                                _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream_ptr(X.device)))
    return out


def qlora_linear_fwd_save(X, W: NF4Weight, A, B, scale: float, ws=None, out=None, hs=None):
    """(Y, Hs): qlora_linear_fwd's Y and the adapter activations Hs =
    bf16(scale X A^T) [M, r] that qlora_linear_bwd_saved takes (r >= 1)."""
    torch = _torch()
    M = _activation("X", X, W)
    K, N = W.cols, W.rows
    r = _adapter(W, A, B, W.device)
    if r == 0:
        raise ValueError("qlora_linear_fwd_save needs an adapter (r >= 1)")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    else:
        _need_cuda("out", out, torch.bfloat16, (M, N), W.device)
    if hs is None:
        hs = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    else:
        _need_cuda("hs", hs, torch.bfloat16, (M, r), W.device)
    ws = _linear_ws(M, N, K, r, X.device, ws)
    st = W.c_struct()
    _check("qlora_linear_fwd_save",
           lib.qlora_linear_fwd_save(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale),
                                     _ptr(out), _ptr(hs), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream_ptr(X.device)))
    return out, hs


def _bwd_outs(M, N, K, r, W, device, outs):
    torch = _torch()
    if outs is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=device)
        dA = torch.empty((r, K), dtype=torch.float32, device=device) if r else None
        dB = torch.empty((N, r), dtype=torch.float32, device=device) if r else None
    else:
        dX, dA, dB = outs
        _need_cuda("dX", dX, torch.bfloat16, (M, K), W.device)
        if r:
            _need_cuda("dA", dA, torch.float32, (r, K), W.device)
            _need_cuda("dB", dB, torch.float32, (N, r), W.device)
        elif dA is not None or dB is not None:
            raise ValueError("without an adapter dA and dB must be None")
    return dX, dA, dB


def qlora_linear_bwd(dY, X, W: NF4Weight, A=None, B=None, scale: float = 0.0, ws=None,
                     outs: Optional[Tuple] = None):
    """(dX, dA, dB) of the QLoRA linear layer; the base weight gets no gradient."""
    torch = _torch()
    M = _activation("X", X, W)
    K, N = W.cols, W.rows
    _need_cuda("dY", dY, torch.bfloat16, (M, N), W.device)
    r = _adapter(W, A, B, W.device)
    dX, dA, dB = _bwd_outs(M, N, K, r, W, X.device, outs)
    ws = _linear_ws(M, N, K, r, X.device, ws)
    st = W.c_struct()
    _check("qlora_linear_bwd",
           lib.qlora_linear_bwd(_ptr(dY), _ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                float(scale), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream_ptr(X.device)))
    return dX, dA, dB


def qlora_linear_bwd_saved(dY, X, Hs, W: NF4Weight, A, B, scale: float, ws=None,
                           outs: Optional[Tuple] = None):
    """qlora_linear_bwd with the Hs of qlora_linear_fwd_save (same X, A and
    scale): the adapter activations are not formed again (r >= 1)."""
    torch = _torch()
    M = _activation("X", X, W)
    K, N = W.cols, W.rows
    _need_cuda("dY", dY, torch.bfloat16, (M, N), W.device)
    r = _adapter(W, A, B, W.device)
    if r == 0:
        raise ValueError("qlora_linear_bwd_saved needs an adapter (r >= 1)")
    _need_cuda("Hs", Hs, torch.bfloat16, (M, r), W.device)
    dX, dA, dB = _bwd_outs(M, N, K, r, W, X.device, outs)
    ws = _linear_ws(M, N, K, r, X.device, ws)
    st = W.c_struct()
    _check("qlora_linear_bwd_saved",
           lib.qlora_linear_bwd_saved(_ptr(dY), _ptr(X), _ptr(Hs), M, ctypes.byref(st), _ptr(A), _ptr(B),
                                      r, float(scale), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream_ptr(X.device)))
    return dX, dA, dB


def qlora_linear_fwd_noalloc(X, W: NF4Weight, A=None, B=None, scale: float = 0.0, out=None):
    """qlora_linear_fwd through the allocation-free entry point: no workspace,
    and ``out`` (bf16 [M, N]) must be given, so nothing is allocated."""
    torch = _torch()
    M = _activation("X", X, W)
    r = _adapter(W, A, B, W.device)
    if out is None:
        raise ValueError("out must be given: the allocation-free call allocates nothing")
    _need_cuda("out", out, torch.bfloat16, (M, W.rows), W.device)
    st = W.c_struct()
    _check("qlora_linear_fwd_noalloc",
           lib.qlora_linear_fwd_noalloc(_ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(scale),
                                        _ptr(out), _stream_ptr(X.device)))
    return out
