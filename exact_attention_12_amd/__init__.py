"""Python binding of libattn.so, the gfx950 exact-attention library.

Argument marshalling only: tensors are checked (device, dtype, shape), their
device pointers, strides and the current HIP stream are passed to the C ABI
declared in include/attn.h, and outputs are allocated with torch. Every step of
the computation runs in the library's HIP kernels; there is no other code path.
If the library is missing or fails to load, every call raises.

    o, lse = fwd(q, k, v, causal=True)              # scale defaults to 1/sqrt(d)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o, lse = fwd(q, k, v, window=256)               # sliding window i-256 < j <= i
    o, lse = fwd(q, k, v, layout="bshd")            # [B, N, H, d] tensors, read in place
    o = attention(q, k, v, causal=True)             # differentiable: o.backward() runs bwd

Tensors are bf16 or fp16 (all of one call alike), 4-D, innermost dim
contiguous; `layout` says whether dims 1 and 2 are (H, N) ("bhsd", default) or
(N, H) ("bshd"). Contiguous bf16 BHSD calls go through attn_fwd / attn_bwd (and
their window and pass variants); anything else through attn_fwd_ex /
attn_bwd_ex with explicit strides.
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

SUPPORTED_HEAD_DIMS = (32, 64, 80, 96, 128, 192, 256)

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
    10: "ATTN_ERR_STRIDE",
    11: "ATTN_ERR_DTYPE",
    12: "ATTN_ERR_PASSES",
    13: "ATTN_ERR_DROPOUT",
    14: "ATTN_ERR_SCRATCH",
}

MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW = 0, 1, 2
DTYPE_BF16, DTYPE_FP16 = 0, 1
PASS_BITS = {"pre": 1, "dkdv": 2, "dq": 4}


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
        ("key_splits", ctypes.c_int),
        ("key_groups", ctypes.c_int),
        ("products16", ctypes.c_int),
    ]


class AttnTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_longlong),
        ("stride_h", ctypes.c_longlong),
        ("stride_n", ctypes.c_longlong),
    ]


class AttnDecodeProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int),
        ("Hq", ctypes.c_int),
        ("Hkv", ctypes.c_int),
        ("Nq", ctypes.c_int),
        ("Nk", ctypes.c_int),
        ("d", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("mask", ctypes.c_int),
        ("window", ctypes.c_int),
        ("dtype", ctypes.c_int),
    ]


class AttnProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int),
        ("Hq", ctypes.c_int),
        ("Hkv", ctypes.c_int),
        ("N", ctypes.c_int),
        ("d", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("mask", ctypes.c_int),
        ("window", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("dropout_p", ctypes.c_float),
        ("seed", ctypes.c_ulonglong),
        ("offset", ctypes.c_uint),
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
    vp, i, f, sz, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint
    tp, pp = ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnProblem)
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd_ex.argtypes = [pp, tp, tp, tp, tp, vp, vp]
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    L.attn_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
    L.attn_bwd_ex.argtypes = [pp, tp, tp, tp, tp, vp, tp, tp, tp, tp, vp, sz, u, vp]
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_bwd_noalloc_max_rows.argtypes = []
    L.attn_bwd_noalloc_max_rows.restype = sz
    L.attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, vp]
    L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    dp = ctypes.POINTER(AttnDecodeProblem)
    L.attn_decode_workspace_bytes.argtypes = [dp]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode_fwd.argtypes = [dp, tp, tp, tp, vp, tp, vp, vp, sz, vp]
    for name in ("attn_decode_fwd", "attn_fwd", "attn_fwd_window", "attn_fwd_ex", "attn_bwd", "attn_bwd_window",
                 "attn_bwd_ex", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq",
                 "attn_bwd_noalloc"):
        getattr(L, name).restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_hip_error.argtypes = []
    L.attn_last_hip_error.restype = ctypes.c_char_p
    L.attn_fwd_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(AttnPlan)]
    L.attn_fwd_plan.restype = i
    L.attn_probe_mfma_src_elems.argtypes = [i]
    L.attn_probe_mfma_src_elems.restype = sz
    L.attn_probe_mfma_rate.argtypes = [vp, vp, i, i, i, vp]
    L.attn_probe_mfma_rate.restype = i
    L.attn_probe_mfma16_rate.argtypes = [vp, vp, i, i, i, vp]
    L.attn_probe_mfma16_rate.restype = i
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    inc = os.path.dirname(HEADER_PATH)
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
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


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_FP16
    raise TypeError(f"tensors must be bfloat16 or float16 (got {t.dtype})")


def _as_bhsd(t, name, layout):
    """The [B, H, N, d] view of a 4-D operand given in `layout`."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims (got shape {tuple(t.shape)})")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")
    if layout == "bhsd":
        return t
    if layout == "bshd":
        return t.transpose(1, 2)
    raise ValueError(f"layout must be 'bhsd' or 'bshd' (got {layout!r})")


def _new_like(ref_bhsd, layout):
    """A fresh output with ref's [B, H, N, d] shape, contiguous in `layout`,
    returned as its [B, H, N, d] view."""
    import torch
    B, H, N, d = ref_bhsd.shape
    if layout == "bshd":
        return torch.empty((B, N, H, d), dtype=ref_bhsd.dtype, device=ref_bhsd.device).transpose(1, 2)
    return torch.empty((B, H, N, d), dtype=ref_bhsd.dtype, device=ref_bhsd.device)


def _plain(ts):
    """True when every tensor is contiguous bf16 [B, H, N, d]."""
    import torch
    return all(t is None or (t.dtype == torch.bfloat16 and t.is_contiguous()) for t in ts)


def _tensor(t):
    if t is None:
        return None
    return ctypes.byref(AttnTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)))


def _shapes(q, k, v):
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must have one dtype")
    _dtype_code(q)
    return B, Hq, k.shape[1], N, d


def _same(t, name, ref):
    if tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} must have shape {tuple(ref.shape)} (got {tuple(t.shape)})")
    if t.dtype != ref.dtype:
        raise TypeError(f"{name} must be {ref.dtype} (got {t.dtype})")
    if t.device != ref.device:
        raise ValueError(f"{name} must be on {ref.device}")


def _rows(t, name, B, Hq, N, device):
    import torch
    if not isinstance(t, torch.Tensor) or t.device != device or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 tensor on {device}")
    if tuple(t.shape) != (B, Hq, N) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, Hq, N] = {(B, Hq, N)}")


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


def _problem(B, Hq, Hkv, N, d, scale, causal, window, dtype, dropout=None):
    if window is not None:
        mask, win = MASK_SLIDING_WINDOW, window
    else:
        mask, win = (MASK_CAUSAL if causal else MASK_NONE), 0
    p, seed, offset = dropout if dropout is not None else (0.0, 0, 0)
    return AttnProblem(B, Hq, Hkv, N, d, float(scale), mask, win, dtype, float(p), int(seed), int(offset))


def _dropout_arg(dropout_p, seed, offset):
    if not dropout_p:
        return None
    if not (0.0 <= float(dropout_p) < 1.0):
        raise ValueError("dropout_p must be in [0, 1)")
    return float(dropout_p), int(seed) & ((1 << 64) - 1), int(offset) & 0xFFFFFFFF


def fwd(q, k, v, *, scale=None, causal=False, window=None, layout="bhsd", out=None, lse=None,
        use_ex=False, dropout_p=0.0, seed=0, offset=0):
    """Forward pass. q [B,Hq,N,d], k, v [B,Hkv,N,d] (dims 1, 2 swapped for
    layout="bshd"), bf16 or fp16, on the GPU.

    window=W (>= 1) selects the sliding-window mask i-W < j <= i, which
    implies the causal mask. Returns (o like q, lse [B,Hq,N] float32).
    Enqueued on the current stream; no synchronisation. use_ex forces the
    strided entry point even for plain tensors. dropout_p > 0 drops attention
    weights with the Philox stream keyed by (seed, offset) (see attn.h).
    """
    import torch
    window = _window_arg(window)
    drop = _dropout_arg(dropout_p, seed, offset)
    qv, kv_, vv = (_as_bhsd(t, n, layout) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    B, Hq, Hkv, N, d = _shapes(qv, kv_, vv)
    if scale is None:
        scale = default_scale(d)
    ov = _new_like(qv, layout) if out is None else _as_bhsd(out, "out", layout)
    _same(ov, "out", qv)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _rows(lse, "lse", B, Hq, N, q.device)
    st = _stream_ptr(q.device)
    L = lib()
    if not use_ex and drop is None and _plain((qv, kv_, vv, ov)):
        if window is None:
            _check(L.attn_fwd(qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), ov.data_ptr(), lse.data_ptr(),
                              B, Hq, Hkv, N, d, float(scale), int(bool(causal)), st))
        else:
            _check(L.attn_fwd_window(qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), ov.data_ptr(),
                                     lse.data_ptr(), B, Hq, Hkv, N, d, float(scale), window, st))
    else:
        prob = _problem(B, Hq, Hkv, N, d, scale, causal, window, _dtype_code(qv), drop)
        _check(L.attn_fwd_ex(ctypes.byref(prob), _tensor(qv), _tensor(kv_), _tensor(vv), _tensor(ov),
                             lse.data_ptr(), st))
    return (ov.transpose(1, 2) if layout == "bshd" else ov), lse


def bwd_workspace_bytes(B, Hq, Hkv, N, d) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def bwd(q, k, v, o, lse, do, *, scale=None, causal=False, window=None, layout="bhsd",
        workspace=None, dq=None, dk=None, dv=None, use_ex=False, dropout_p=0.0, seed=0, offset=0):
    """Backward pass; returns (dq, dk, dv) like q, k, v. `causal`, `window`,
    `layout` and the dropout arguments must be those of the forward call."""
    return bwd_passes(q, k, v, o, lse, do, dq, dk, dv, workspace, scale=scale, causal=causal,
                      window=window, layout=layout, passes=("pre", "dkdv", "dq"), use_ex=use_ex,
                      fused=True, dropout_p=dropout_p, seed=seed, offset=offset)


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, *, scale=None, causal=False):
    """attn_bwd_noalloc: the backward with the library's fixed scratch in
    place of a workspace (contiguous bf16 BHSD tensors; dq, dk, dv are the
    caller's outputs, written in place). Nothing is allocated on the device,
    by torch or by the library."""
    import torch
    qv, kv_, vv = (_as_bhsd(t, n, "bhsd") for t, n in ((q, "q"), (k, "k"), (v, "v")))
    B, Hq, Hkv, N, d = _shapes(qv, kv_, vv)
    for name, t, ref in (("o", o, qv), ("do", do, qv), ("dq", dq, qv), ("dk", dk, kv_), ("dv", dv, vv)):
        _same(_as_bhsd(t, name, "bhsd"), name, ref)
    _rows(lse, "lse", B, Hq, N, q.device)
    ts = (qv, kv_, vv, o, do, dq, dk, dv)
    if qv.dtype != torch.bfloat16 or not _plain(ts):
        raise ValueError("bwd_noalloc takes contiguous bfloat16 [B, H, N, d] tensors")
    if scale is None:
        scale = default_scale(d)
    _check(lib().attn_bwd_noalloc(qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                  _stream_ptr(q.device)))
    return dq, dk, dv


def bwd_noalloc_max_rows() -> int:
    return int(lib().attn_bwd_noalloc_max_rows())


def bwd_passes(q, k, v, o, lse, do, dq, dk, dv, workspace, *, scale=None, causal=False,
               window=None, layout="bhsd", passes=("pre", "dkdv", "dq"), use_ex=False, fused=False,
               dropout_p=0.0, seed=0, offset=0):
    """Run selected backward passes (same arguments and checks as bwd()). With
    fused=False each pass goes through its own entry point; outputs may be
    None and are then allocated. A window implies the causal mask."""
    import torch
    window = _window_arg(window)
    drop = _dropout_arg(dropout_p, seed, offset)
    if window is not None:
        causal = True
    bits = 0
    for p in passes:
        if p not in PASS_BITS:
            raise ValueError(f"unknown backward pass {p!r}")
        bits |= PASS_BITS[p]
    qv, kv_, vv = (_as_bhsd(t, n, layout) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    B, Hq, Hkv, N, d = _shapes(qv, kv_, vv)
    ov, dov = _as_bhsd(o, "o", layout), _as_bhsd(do, "do", layout)
    _same(ov, "o", qv)
    _same(dov, "do", qv)
    _rows(lse, "lse", B, Hq, N, q.device)
    if scale is None:
        scale = default_scale(d)
    outs = []
    for name, t, ref in (("dq", dq, qv), ("dk", dk, kv_), ("dv", dv, vv)):
        tv = _new_like(ref, layout) if t is None else _as_bhsd(t, name, layout)
        _same(tv, name, ref)
        outs.append(tv)
    dqv, dkv, dvv = outs
    need = bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = _stream_ptr(q.device)
    L = lib()
    win = 0 if window is None else window
    if not use_ex and drop is None and _plain((qv, kv_, vv, ov, dov, dqv, dkv, dvv)):
        args = (qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), ov.data_ptr(), lse.data_ptr(),
                dov.data_ptr(), dqv.data_ptr(), dkv.data_ptr(), dvv.data_ptr(), ws, wsb,
                B, Hq, Hkv, N, d, float(scale))
        if fused and bits == 7:
            if window is None:
                _check(L.attn_bwd(*args, int(bool(causal)), st))
            else:
                _check(L.attn_bwd_window(*args, window, st))
        else:
            for p in ("pre", "dkdv", "dq"):
                if not bits & PASS_BITS[p]:
                    continue
                if p == "pre":
                    _check(L.attn_bwd_preprocess(ov.data_ptr(), dov.data_ptr(), lse.data_ptr(), ws, wsb,
                                                 B, Hq, Hkv, N, d, st))
                elif p == "dkdv":
                    _check(L.attn_bwd_dkdv(qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), lse.data_ptr(),
                                           dov.data_ptr(), dkv.data_ptr(), dvv.data_ptr(), ws, wsb,
                                           B, Hq, Hkv, N, d, float(scale), int(bool(causal)), win, st))
                else:
                    _check(L.attn_bwd_dq(qv.data_ptr(), kv_.data_ptr(), vv.data_ptr(), lse.data_ptr(),
                                         dov.data_ptr(), dqv.data_ptr(), ws, wsb,
                                         B, Hq, Hkv, N, d, float(scale), int(bool(causal)), win, st))
    else:
        prob = _problem(B, Hq, Hkv, N, d, scale, causal, window, _dtype_code(qv), drop)
        _check(L.attn_bwd_ex(ctypes.byref(prob), _tensor(qv), _tensor(kv_), _tensor(vv), _tensor(ov),
                             lse.data_ptr(), _tensor(dov), _tensor(dqv), _tensor(dkv), _tensor(dvv),
                             ws, wsb, bits, st))
    if layout == "bshd":
        return tuple(t.transpose(1, 2) for t in outs)
    return dqv, dkv, dvv


_ATTENTION_FN = None


def _attention_fn():
    """The torch.autograd.Function behind attention(), built on first use (the
    module itself does not import torch)."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        import torch

        class AttentionFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal, window, layout, dropout_p, seed, offset):
                o, lse = fwd(q, k, v, scale=scale, causal=causal, window=window, layout=layout,
                             dropout_p=dropout_p, seed=seed, offset=offset)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.args = (scale, causal, window, layout, dropout_p, seed, offset)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                scale, causal, window, layout, dropout_p, seed, offset = ctx.args
                # the incoming gradient may be a broadcast or otherwise strided view
                dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), scale=scale, causal=causal,
                                 window=window, layout=layout, dropout_p=dropout_p, seed=seed,
                                 offset=offset)
                return dq, dk, dv, None, None, None, None, None, None, None

        _ATTENTION_FN = AttentionFn
    return _ATTENTION_FN


def attention(q, k, v, *, scale=None, causal=False, window=None, layout="bhsd", dropout_p=0.0,
              seed=None, offset=0):
    """Differentiable attention: fwd() as a torch autograd function whose
    backward is bwd() (the same kernels, nothing recomputed on the host).
    Arguments as for fwd(); returns O only (the LSE is kept for the backward).
    With dropout_p > 0 and no seed, a seed is drawn from torch's default
    generator, and the backward redraws the same keep mask from it."""
    if scale is None:
        scale = default_scale(q.shape[-1])
    if dropout_p and seed is None:
        import torch
        seed = int(torch.randint(0, 2 ** 31 - 1, (1,)).item())
    return _attention_fn().apply(q, k, v, float(scale), causal, window, layout, float(dropout_p),
                                 0 if seed is None else int(seed), int(offset))


def _decode_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window, dtype):
    if window is not None:
        mask, win = MASK_SLIDING_WINDOW, window
    else:
        mask, win = (MASK_CAUSAL if causal else MASK_NONE), 0
    return AttnDecodeProblem(B, Hq, Hkv, Nq, Nk, d, float(scale), mask, win, dtype)


def decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal=False, window=None, dtype=DTYPE_BF16) -> int:
    prob = _decode_problem(B, Hq, Hkv, Nq, Nk, d, 1.0, causal, window, dtype)
    return int(lib().attn_decode_workspace_bytes(ctypes.byref(prob)))


def decode(q, k_cache, v_cache, *, kv_lens=None, scale=None, causal=False, window=None,
           layout="bhsd", out=None, lse=None, workspace=None):
    """Attention of Nq new queries per sequence against a KV cache.

    q [B,Hq,Nq,d]; k_cache, v_cache [B,Hkv,Nk,d] (dims 1, 2 swapped for
    layout="bshd"); kv_lens: None (every sequence fills the cache) or an
    int32 GPU tensor [B] of valid cache rows. Query i of sequence b is the
    token at position kv_lens[b] - Nq + i. Returns (o like q, lse [B,Hq,Nq]).
    """
    import torch
    window = _window_arg(window)
    qv = _as_bhsd(q, "q", layout)
    kv_, vv = _as_bhsd(k_cache, "k_cache", layout), _as_bhsd(v_cache, "v_cache", layout)
    B, Hq, Nq, d = qv.shape
    if kv_.shape != vv.shape or kv_.shape[0] != B or kv_.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(qv.shape)}, caches {tuple(kv_.shape)}, {tuple(vv.shape)}")
    if not (qv.dtype == kv_.dtype == vv.dtype):
        raise TypeError("q and the caches must have one dtype")
    Hkv, Nk = kv_.shape[1], kv_.shape[2]
    if scale is None:
        scale = default_scale(d)
    ov = _new_like(qv, layout) if out is None else _as_bhsd(out, "out", layout)
    _same(ov, "out", qv)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _rows(lse, "lse", B, Hq, Nq, q.device)
    lens_ptr = None
    if kv_lens is not None:
        if (not isinstance(kv_lens, torch.Tensor) or kv_lens.dtype != torch.int32
                or kv_lens.device != q.device or tuple(kv_lens.shape) != (B,) or not kv_lens.is_contiguous()):
            raise TypeError("kv_lens must be a contiguous int32 tensor [B] on the GPU")
        lens_ptr = kv_lens.data_ptr()
    prob = _decode_problem(B, Hq, Hkv, Nq, Nk, d, scale, causal, window, _dtype_code(qv))
    L = lib()
    need = int(L.attn_decode_workspace_bytes(ctypes.byref(prob)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.attn_decode_fwd(ctypes.byref(prob), _tensor(qv), _tensor(kv_), _tensor(vv), lens_ptr,
                             _tensor(ov), lse.data_ptr(), ws, wsb, _stream_ptr(q.device)))
    return (ov.transpose(1, 2) if layout == "bshd" else ov), lse


def fwd_plan(B, Hq, Hkv, N, d, causal=False) -> dict:
    plan = AttnPlan()
    _check(lib().attn_fwd_plan(B, Hq, Hkv, N, d, int(bool(causal)), ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in AttnPlan._fields_}


def probe_mfma_rate(src, dst, blocks, iters, chains=8, shape="32x32x16"):
    """attn_probe_mfma_rate or, for shape "16x16x32", attn_probe_mfma16_rate
    (include/attn_probe.h): enqueue the matrix-core rate probe on the current
    stream; src holds probe_mfma_src_elems(blocks) bf16 values, dst
    blocks * 512 floats. Returns the flops it enqueues (the same for both
    shapes)."""
    import torch
    if src.dtype != torch.bfloat16 or src.numel() < lib().attn_probe_mfma_src_elems(blocks):
        raise ValueError("src must hold probe_mfma_src_elems(blocks) bf16 values")
    if dst.dtype != torch.float32 or dst.numel() < blocks * 512:
        raise ValueError("dst must hold blocks * 512 floats")
    fn = {"32x32x16": lib().attn_probe_mfma_rate, "16x16x32": lib().attn_probe_mfma16_rate}.get(shape)
    if fn is None:
        raise ValueError("shape must be '32x32x16' or '16x16x32'")
    _check(fn(src.data_ptr(), dst.data_ptr(), blocks, iters, chains, _stream_ptr(src.device)))
    return blocks * 8 * 8 * iters * 32768.0


def probe_mfma_src_elems(blocks) -> int:
    return int(lib().attn_probe_mfma_src_elems(blocks))
