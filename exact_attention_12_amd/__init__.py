"""Python binding of libattn.so, the gfx950 exact-attention library.

Argument marshalling only: tensors are checked (device, dtype, layout), their
device pointers and the current HIP stream are passed to the C ABI declared in
include/attn.h, and outputs are allocated with torch. Every step of the
computation runs in the library's HIP kernels; there is no other code path.
If the library is missing or fails to load, every call raises.

    o, lse = fwd(q, k, v, causal=True)              # scale defaults to 1/sqrt(d)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o, lse = fwd(q, k, v, window=256)               # sliding window i-256 < j <= i
"""

from __future__ import annotations

import ctypes
import math
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT_DIR = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
HEADER_PATH = os.path.join(ROOT_DIR, "include", "attn.h")

SUPPORTED_HEAD_DIMS = (64, 80, 128, 256)

STATUS = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_GQA",
    4: "ATTN_ERR_HEAD_DIM",
    5: "ATTN_ERR_SCALE",
    6: "ATTN_ERR_ALIGN",
    7: "ATTN_ERR_WORKSPACE",
    8: "ATTN_ERR_HIP",
    9: "ATTN_ERR_WINDOW",
}


class AttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.name = STATUS.get(code, str(code))


class AttnPlan(ctypes.Structure):
    _fields_ = [
        ("rows_per_wave", ctypes.c_int),
        ("block_q", ctypes.c_int),
        ("block_kv", ctypes.c_int),
        ("threads", ctypes.c_int),
        ("workgroups", ctypes.c_longlong),
        ("lds_bytes", ctypes.c_int),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn.so (built by exact_attention_12_amd.build) once."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_12_amd.build` "
            "or __graft_entry__.build(); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd_window.restype = i
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    L.attn_bwd_window.restype = i
    L.attn_bwd_preprocess.argtypes = [vp, vp, vp, sz, i, i, i, i, i, vp]
    L.attn_bwd_preprocess.restype = i
    L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    L.attn_bwd_dkdv.restype = i
    L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    L.attn_bwd_dq.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_hip_error.argtypes = []
    L.attn_last_hip_error.restype = ctypes.c_char_p
    L.attn_fwd_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(AttnPlan)]
    L.attn_fwd_plan.restype = i
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/attn.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(attn_\w+)\s*\(", text, re.M)))


def status_string(code: int) -> str:
    return lib().attn_status_string(code).decode()


def _check(code: int):
    if code != 0:
        msg = status_string(code)
        if code == 8:
            msg += ": " + lib().attn_last_hip_error().decode()
        raise AttnError(code, msg)


def _stream_ptr(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _require(t, name, dtype, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _shapes(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, 4)
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    return B, Hq, k.shape[1], N, d


def default_scale(d: int) -> float:
    """1/sqrt(d), the scale of the standard attention formula."""
    return 1.0 / math.sqrt(d)


def _window_arg(window):
    if window is None:
        return None
    window = int(window)
    if window < 1:
        raise ValueError("window must be >= 1")
    return window


def fwd(q, k, v, *, scale=None, causal=False, window=None, out=None, lse=None):
    """Forward pass. q [B,Hq,N,d], k, v [B,Hkv,N,d] bf16 contiguous on the GPU.

    window=W (>= 1) selects the sliding-window mask i-W < j <= i, which
    implies the causal mask. Returns (o [B,Hq,N,d] bf16, lse [B,Hq,N] float32).
    Enqueued on the current stream; no synchronisation.
    """
    window = _window_arg(window)
    import torch
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", torch.bfloat16, 4)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    else:
        _require(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, N):
            raise ValueError("lse must be [B, Hq, N]")
    if window is None:
        _check(lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _stream_ptr(q.device)))
    else:
        _check(lib().attn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, Hq, Hkv, N, d, float(scale), window,
                                     _stream_ptr(q.device)))
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, N, d) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def bwd(q, k, v, o, lse, do, *, scale=None, causal=False, window=None, workspace=None,
        dq=None, dk=None, dv=None):
    """Backward pass; returns (dq, dk, dv) bf16 like q, k, v. `causal` and
    `window` must be those of the forward call."""
    import torch
    window = _window_arg(window)
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    _require(o, "o", torch.bfloat16, 4)
    _require(do, "do", torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    if o.shape != q.shape or do.shape != q.shape or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o, do must have the shape of q and lse must be [B, Hq, N]")
    if scale is None:
        scale = default_scale(d)
    need = bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _require(t, name, torch.bfloat16, 4)
        if t.shape != ref.shape:
            raise ValueError(f"{name} has the wrong shape")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            B, Hq, Hkv, N, d, float(scale))
    if window is None:
        _check(lib().attn_bwd(*args, int(bool(causal)), _stream_ptr(q.device)))
    else:
        _check(lib().attn_bwd_window(*args, window, _stream_ptr(q.device)))
    return dq, dk, dv


def bwd_passes(q, k, v, o, lse, do, dq, dk, dv, workspace, *, scale=None, causal=False,
               window=None, passes=("pre", "dkdv", "dq")):
    """Run selected backward passes through their own entry points (same
    arguments and checks as bwd(); outputs must be preallocated). A window
    implies the causal mask."""
    import torch
    window = _window_arg(window)
    if window is not None:
        causal = True
    win = 0 if window is None else window
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    if scale is None:
        scale = default_scale(d)
    for name, t in (("o", o), ("do", do), ("dq", dq)):
        _require(t, name, torch.bfloat16, 4)
    for name, t in (("dk", dk), ("dv", dv)):
        _require(t, name, torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    L = lib()
    ws, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = _stream_ptr(q.device)
    for p in passes:
        if p == "pre":
            _check(L.attn_bwd_preprocess(o.data_ptr(), do.data_ptr(), ws, wsb, B, Hq, Hkv, N, d, st))
        elif p == "dkdv":
            _check(L.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), ws, wsb, B, Hq, Hkv, N, d, float(scale),
                                   int(bool(causal)), win, st))
        elif p == "dq":
            _check(L.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                 dq.data_ptr(), ws, wsb, B, Hq, Hkv, N, d, float(scale),
                                 int(bool(causal)), win, st))
        else:
            raise ValueError(f"unknown backward pass {p!r}")
    return dq, dk, dv


def fwd_plan(B, Hq, Hkv, N, d, causal=False) -> dict:
    plan = AttnPlan()
    _check(lib().attn_fwd_plan(B, Hq, Hkv, N, d, int(bool(causal)), ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in AttnPlan._fields_}
