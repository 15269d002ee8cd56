"""The C-ABI library loads, exports every declared symbol, and validates its
arguments on the host (every error code, no device call made)."""

import ctypes
import math

import pytest

import exact_attention_12_amd as ea
from exact_attention_12_amd import build as ea_build


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(ea.LIB_PATH):
        ea_build.build()
    return ea.lib()


P = 0x10000  # fake, aligned, never dereferenced: validation fails before any device call


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125, causal=0):
    return L.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, None)


def bwd(L, ws=P, ws_bytes=1 << 20, ptrs=None, B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125):
    p = ptrs or [P] * 9
    return L.attn_bwd(*p, ws, ws_bytes, B, Hq, Hkv, N, d, scale, 1, None)


def test_exports_every_declared_function(L):
    names = ea.header_functions()
    assert set(names) >= {"attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_string",
                          "attn_last_hip_error", "attn_fwd_plan", "attn_fwd_window",
                          "attn_bwd_window", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(10):
        s = ea.status_string(code)
        assert s and s != "unknown status"
    assert ea.status_string(99) == "unknown status"
    assert L.attn_last_hip_error() == b""


@pytest.mark.parametrize("which", range(5))
def test_fwd_null_pointer(L, which):
    args = [P] * 5
    args[which] = None
    assert fwd(L, *args) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0), dict(Hkv=0), dict(N=0), dict(N=-5),
                                dict(N=(1 << 24) + 1), dict(B=1 << 30, Hq=1 << 30)])
def test_fwd_bad_shape(L, kw):
    assert fwd(L, **kw) == 2


@pytest.mark.parametrize("Hq,Hkv", [(3, 2), (8, 3), (1, 2)])
def test_fwd_bad_grouping(L, Hq, Hkv):
    assert fwd(L, Hq=Hq, Hkv=Hkv) == 3


@pytest.mark.parametrize("d", [0, 32, 63, 96, 112, 160, 192, 512])
def test_fwd_unsupported_head_dim(L, d):
    """Unsupported head dims are rejected with an error rather than served by a
    slower generic path (datacanvas head-dim article: the symptoms section)."""
    assert fwd(L, d=d) == 4


@pytest.mark.parametrize("scale", [0.0, -1.0, math.inf, math.nan, -0.0])
def test_fwd_bad_scale(L, scale):
    assert fwd(L, scale=scale) == 5


@pytest.mark.parametrize("which", range(5))
def test_fwd_misaligned(L, which):
    args = [P] * 5
    args[which] = P + 2
    assert fwd(L, *args) == 6


def test_bwd_errors(L):
    need = L.attn_bwd_workspace_bytes(1, 2, 1, 8, 64)
    assert need == 256
    assert bwd(L, ws=None) == 7
    assert bwd(L, ws_bytes=need - 1) == 7
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert bwd(L, ptrs=ptrs) == 1
        ptrs[i] = P + 4
        assert bwd(L, ptrs=ptrs) == 6
    assert bwd(L, ws=P + 8) == 6
    assert bwd(L, d=96) == 4
    assert bwd(L, Hq=3, Hkv=2) == 3
    assert bwd(L, scale=float("nan")) == 5
    assert bwd(L, N=0) == 2


def test_workspace_bytes(L):
    assert L.attn_bwd_workspace_bytes(1, 16, 16, 16384, 128) == 16 * 16384 * 4
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 1, 64) == 256
    assert L.attn_bwd_workspace_bytes(2, 3, 1, 100, 80) == 2560  # 2400 rounded up to 256
    assert L.attn_bwd_workspace_bytes(1, 3, 2, 100, 80) == 0
    assert L.attn_bwd_workspace_bytes(1, 2, 2, 100, 96) == 0


def test_fwd_plan(L):
    p = ea.fwd_plan(1, 8, 8, 400, 64)
    assert p["block_q"] == 128 and p["threads"] == 256
    assert p["workgroups"] == math.ceil(400 / 128) * 8
    assert p["lds_bytes"] <= 160 * 1024
    for d in ea.SUPPORTED_HEAD_DIMS:
        q = ea.fwd_plan(2, 32, 32, 4096, d, True)
        assert q["workgroups"] == 2 * 32 * 4096 // q["block_q"]
        assert q["lds_bytes"] <= 160 * 1024 // (1 if d == 256 else 2)
    with pytest.raises(ea.AttnError) as e:
        ea.fwd_plan(1, 8, 8, 400, 96)
    assert e.value.name == "ATTN_ERR_HEAD_DIM"


def test_pass_entry_points_validate(L):
    ws, wsb = P, 1 << 20
    # preprocess: o, dout, workspace
    assert L.attn_bwd_preprocess(None, P, ws, wsb, 1, 2, 1, 8, 64, None) == 1
    assert L.attn_bwd_preprocess(P, None, ws, wsb, 1, 2, 1, 8, 64, None) == 1
    assert L.attn_bwd_preprocess(P, P, None, wsb, 1, 2, 1, 8, 64, None) == 7
    assert L.attn_bwd_preprocess(P, P + 2, ws, wsb, 1, 2, 1, 8, 64, None) == 6
    assert L.attn_bwd_preprocess(P, P, ws, 4, 1, 2, 1, 8, 64, None) == 7
    assert L.attn_bwd_preprocess(P, P, ws, wsb, 1, 2, 1, 8, 96, None) == 4
    # dK/dV pass: q, k, v, lse, dout, dk, dv, workspace
    for i in range(7):
        a = [P] * 7
        a[i] = None
        assert L.attn_bwd_dkdv(*a, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, 0, None) == 1
        a[i] = P + 8
        assert L.attn_bwd_dkdv(*a, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, 0, None) == 6
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 2, 1, 8, 64, -1.0, 1, 0, None) == 5
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 3, 2, 8, 64, 0.125, 1, 0, None) == 3
    # dQ pass: q, k, v, lse, dout, dq, workspace
    for i in range(6):
        a = [P] * 6
        a[i] = None
        assert L.attn_bwd_dq(*a, ws, wsb, 1, 2, 1, 8, 64, 0.125, 0, 0, None) == 1
    assert L.attn_bwd_dq(*[P] * 6, None, wsb, 1, 2, 1, 8, 64, 0.125, 0, 0, None) == 7
    assert L.attn_bwd_dq(*[P] * 6, ws, wsb, 1, 2, 1, 0, 64, 0.125, 0, 0, None) == 2


def test_window_validation(L):
    """The sliding-window mask needs W >= 1 and implies the causal mask (CANN
    FlashAttention page, tuning section on mask modes)."""
    for w in (0, -1, -(1 << 30)):
        assert L.attn_fwd_window(*[P] * 5, 1, 2, 1, 8, 64, 0.125, w, None) == 9
        assert L.attn_bwd_window(*[P] * 10, 1 << 20, 1, 2, 1, 8, 64, 0.125, w, None) == 9
    # the window is checked before anything else in the window entry points
    assert L.attn_fwd_window(None, *[P] * 4, 1, 2, 1, 8, 64, 0.125, 0, None) == 9
    # valid windows still get the ordinary checks
    assert L.attn_fwd_window(None, *[P] * 4, 1, 2, 1, 8, 64, 0.125, 3, None) == 1
    assert L.attn_fwd_window(*[P] * 5, 1, 2, 1, 8, 96, 0.125, 3, None) == 4
    assert L.attn_fwd_window(*[P] * 4, P + 2, 1, 2, 1, 8, 64, 0.125, 1 << 30, None) == 6
    assert L.attn_bwd_window(*[P] * 10, 16, 1, 2, 1, 8, 64, 0.125, 4, None) == 7
    assert L.attn_bwd_window(*[P] * 10, 1 << 20, 1, 2, 1, 8, 64, float("inf"), 4, None) == 5
    # pass entry points: window >= 1 needs causal, negative windows are refused
    ws, wsb = P, 1 << 20
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 2, 1, 8, 64, 0.125, 0, 4, None) == 9
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, -1, None) == 9
    assert L.attn_bwd_dq(*[P] * 6, ws, wsb, 1, 2, 1, 8, 64, 0.125, 0, 2, None) == 9
    assert L.attn_bwd_dq(*[P] * 6, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, -3, None) == 9
