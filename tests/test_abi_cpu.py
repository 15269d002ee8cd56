"""The C-ABI library loads, exports every declared symbol, and validates its
arguments on the host (every error code, no device call made)."""

import ctypes
import math

import pytest
import torch

import exact_attention_12_amd as ea
from exact_attention_12_amd import build as ea_build


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(ea.LIB_PATH):
        ea_build.build()
    return ea.lib()


P = 0x10000  # fake, aligned, never dereferenced: validation fails before any device call

# Every call here must fail validation; should one pass by mistake it would
# launch kernels on the fake pointers, so the module never runs next to a GPU.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only checks with fake device pointers")


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
    for code in range(15):
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
                                dict(N=(1 << 24) + 1), dict(B=1 << 30, Hq=1 << 30),
                                dict(Hq=1 << 15, Hkv=1, N=1 << 16),
                                dict(B=2, Hq=1 << 14, Hkv=1, N=(1 << 16) - 100)])
def test_fwd_bad_shape(L, kw):
    assert fwd(L, **kw) == 2


@pytest.mark.parametrize("kw", [dict(Hq=1 << 15, Hkv=1, N=1 << 16),
                                dict(B=1 << 10, Hq=1 << 5, Hkv=1, N=(1 << 16) - 255)])
def test_bwd_rows_past_the_grid_limit(L, kw):
    # B * Hq * round_up(N, 256) >= 2^31 rows: two work-items per row would
    # pass the 2^32 work-items of one grid dimension
    assert bwd(L, **kw) == 2


@pytest.mark.parametrize("Hq,Hkv", [(3, 2), (8, 3), (1, 2)])
def test_fwd_bad_grouping(L, Hq, Hkv):
    assert fwd(L, Hq=Hq, Hkv=Hkv) == 3


@pytest.mark.parametrize("d", [0, 16, 48, 63, 100, 112, 160, 224, 320, 512])
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
    assert need == 512  # D_i and base-2 LSE, 256 bytes each
    assert bwd(L, ws=None) == 7
    assert bwd(L, ws_bytes=need - 1) == 7
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert bwd(L, ptrs=ptrs) == 1
        ptrs[i] = P + 4
        assert bwd(L, ptrs=ptrs) == 6
    assert bwd(L, ws=P + 8) == 6
    assert bwd(L, d=112) == 4
    assert bwd(L, Hq=3, Hkv=2) == 3
    assert bwd(L, scale=float("nan")) == 5
    assert bwd(L, N=0) == 2


def test_workspace_bytes(L):
    assert L.attn_bwd_workspace_bytes(1, 16, 16, 16384, 128) == 2 * 16 * 16384 * 4
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 1, 64) == 512
    assert L.attn_bwd_workspace_bytes(2, 3, 1, 100, 80) == 2 * 2560  # 2400 rounded up to 256, twice
    # d = 128 with 256 .. 511 blocks of 256 keys and an even group size: the
    # dK/dV pass also keeps fp32 partial dK and dV of two head halves
    assert L.attn_bwd_workspace_bytes(1, 64, 8, 8192, 128) == 2 * 64 * 8192 * 4 + 2 * 2 * 8 * 8192 * 128 * 4
    assert L.attn_bwd_workspace_bytes(1, 64, 8, 8192, 64) == 2 * 64 * 8192 * 4
    assert L.attn_bwd_workspace_bytes(1, 8, 8, 8192, 128) == 2 * 8 * 8192 * 4  # G = 1: no split
    assert L.attn_bwd_workspace_bytes(1, 3, 2, 100, 80) == 0
    # small grids (B * Hkv * ceil(N / 128) <= 256, N >= 512, d <= 128, no
    # 64-key form): two workgroups per 128-key block, fp32 partials
    rt = lambda B, Hq, N: 2 * (-(-B * Hq * N * 4 // 256) * 256)
    assert L.attn_bwd_workspace_bytes(1, 2, 2, 4096, 128) == rt(1, 2, 4096) + 2 * 2 * 2 * 4096 * 128 * 4
    assert L.attn_bwd_workspace_bytes(1, 4, 4, 4096, 80) == rt(1, 4, 4096) + 2 * 2 * 4 * 4096 * 80 * 4
    assert L.attn_bwd_workspace_bytes(1, 16, 16, 4096, 80) == rt(1, 16, 4096)   # 512 blocks: none
    assert L.attn_bwd_workspace_bytes(1, 4, 4, 511, 64) == rt(1, 4, 511)        # N < 512: none
    assert L.attn_bwd_workspace_bytes(1, 2, 2, 4096, 192) == rt(1, 2, 4096)     # d > 128: none
    assert L.attn_bwd_workspace_bytes(1, 2, 2, 100, 112) == 0


def test_fwd_plan(L):
    # the 20x20-map shape: its 32 workgroups of 128 rows would idle most CUs,
    # so each 32-row query tile gets a workgroup whose 8 waves split the keys
    p = ea.fwd_plan(1, 8, 8, 400, 64)
    assert p["block_q"] == 32 and p["key_splits"] == 8 and p["threads"] == 512
    assert p["workgroups"] == math.ceil(400 / 32) * 8
    assert p["lds_bytes"] <= 160 * 1024
    # past 512 keys, 128 or more workgroups of 128 rows, or d = 128: the step
    # loop with one group of 4 waves
    p = ea.fwd_plan(4, 16, 16, 512, 64)
    assert p["key_splits"] == 1 and p["key_groups"] == 1 and p["block_q"] == 128 and p["threads"] == 256
    # grids so small that the longest block's key tiles are about twice the
    # average SIMD's wave steps or more: two groups of 2 waves over 64 rows,
    # one workgroup per CU
    for shape in [(1, 8, 8, 513, 64), (1, 8, 8, 400, 128), (1, 2, 2, 4096, 128, True), (1, 8, 8, 2048, 128, True)]:
        p = ea.fwd_plan(*shape)
        assert p["key_splits"] == 1 and p["key_groups"] == 2, shape
        assert p["block_q"] == 64 and p["threads"] == 256, shape
        assert p["workgroups"] == math.ceil(shape[3] / 64) * shape[0] * shape[1], shape
        assert p["lds_bytes"] <= 160 * 1024, shape
    assert ea.fwd_plan(1, 8, 8, 2048, 80, True)["lds_bytes"] == 2 * 2 * 64 * (88 + 96) * 2
    # larger grids (the d = 80 training shape among them), head dims past 128: one group
    for shape in [(2, 32, 32, 4096, 128, True), (1, 16, 16, 16384, 128, True), (1, 64, 8, 8192, 128, True),
                  (4, 16, 16, 2048, 64, False), (1, 16, 16, 4096, 80, True), (1, 16, 16, 4096, 128, True),
                  (1, 2, 2, 4096, 192, True), (1, 2, 2, 4096, 256, False)]:
        assert ea.fwd_plan(*shape)["key_groups"] == 1, shape
    # d = 128 on those grids: the 16x16x32 step loop, 128-row workgroups of 4 waves;
    # other head dims: 8 waves on 32x32x16 products
    for shape in [(2, 32, 32, 4096, 128, True), (1, 16, 16, 16384, 128, True), (1, 64, 8, 8192, 128, True),
                  (2, 64, 8, 1024, 128, False)]:
        p = ea.fwd_plan(*shape)
        assert p["products16"] == 1 and p["threads"] == 256 and p["block_q"] == 128, shape
        assert p["lds_bytes"] == 2 * 64 * (144 + 144) * 2, shape
    for shape in [(2, 32, 32, 4096, 64, True), (2, 32, 32, 4096, 80, True), (1, 32, 32, 1000, 128, True),
                  (1, 8, 8, 400, 128)]:
        assert ea.fwd_plan(*shape)["products16"] == 0, shape
    for N, nw in [(1, 2), (64, 2), (128, 2), (129, 4), (256, 4), (257, 8), (512, 8)]:
        assert ea.fwd_plan(1, 2, 1, N, 80, True)["key_splits"] == nw, N
    for d in ea.SUPPORTED_HEAD_DIMS:
        q = ea.fwd_plan(2, 32, 32, 4096, d, True)
        assert q["workgroups"] == 2 * 32 * 4096 // q["block_q"]
        assert q["lds_bytes"] <= 160 * 1024 // (1 if d == 256 else 2)
    with pytest.raises(ea.AttnError) as e:
        ea.fwd_plan(1, 8, 8, 400, 112)
    assert e.value.name == "ATTN_ERR_HEAD_DIM"


def test_pass_entry_points_validate(L):
    ws, wsb = P, 1 << 20
    # preprocess: o, dout, lse, workspace
    assert L.attn_bwd_preprocess(None, P, P, ws, wsb, 1, 2, 1, 8, 64, None) == 1
    assert L.attn_bwd_preprocess(P, None, P, ws, wsb, 1, 2, 1, 8, 64, None) == 1
    assert L.attn_bwd_preprocess(P, P, None, ws, wsb, 1, 2, 1, 8, 64, None) == 1
    assert L.attn_bwd_preprocess(P, P, P, None, wsb, 1, 2, 1, 8, 64, None) == 7
    assert L.attn_bwd_preprocess(P, P + 2, P, ws, wsb, 1, 2, 1, 8, 64, None) == 6
    assert L.attn_bwd_preprocess(P, P, P + 4, ws, wsb, 1, 2, 1, 8, 64, None) == 6
    assert L.attn_bwd_preprocess(P, P, P, ws, 4, 1, 2, 1, 8, 64, None) == 7
    assert L.attn_bwd_preprocess(P, P, P, ws, wsb, 1, 2, 1, 8, 112, None) == 4
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
    assert L.attn_fwd_window(*[P] * 5, 1, 2, 1, 8, 48, 0.125, 3, None) == 4
    assert L.attn_fwd_window(*[P] * 4, P + 2, 1, 2, 1, 8, 64, 0.125, 1 << 30, None) == 6
    assert L.attn_bwd_window(*[P] * 10, 16, 1, 2, 1, 8, 64, 0.125, 4, None) == 7
    assert L.attn_bwd_window(*[P] * 10, 1 << 20, 1, 2, 1, 8, 64, float("inf"), 4, None) == 5
    # pass entry points: window >= 1 needs causal, negative windows are refused
    ws, wsb = P, 1 << 20
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 2, 1, 8, 64, 0.125, 0, 4, None) == 9
    assert L.attn_bwd_dkdv(*[P] * 7, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, -1, None) == 9
    assert L.attn_bwd_dq(*[P] * 6, ws, wsb, 1, 2, 1, 8, 64, 0.125, 0, 2, None) == 9
    assert L.attn_bwd_dq(*[P] * 6, ws, wsb, 1, 2, 1, 8, 64, 0.125, 1, -3, None) == 9


# ------------------------------------------------------------ strided/typed ABI

def T(data=P, sb=1 << 12, sh=1 << 10, sn=64):
    return ea.AttnTensor(data, sb, sh, sn)


def prob(**kw):
    base = dict(B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125, mask=ea.MASK_CAUSAL, window=0,
                dtype=ea.DTYPE_BF16, dropout_p=0.0, seed=0, offset=0)
    base.update(kw)
    return ea.AttnProblem(*[base[f] for f, _ in ea.AttnProblem._fields_])


def fwd_ex(L, pr=None, ts=None, lse=P):
    ts = ts or [T() for _ in range(4)]
    return L.attn_fwd_ex(ctypes.byref(pr or prob()), *[ctypes.byref(t) if t is not None else None
                                                       for t in ts], lse, None)


def bwd_ex(L, pr=None, ts=None, lse=P, ws=P, wsb=1 << 20, passes=7):
    ts = ts if ts is not None else [T() for _ in range(8)]
    r = [ctypes.byref(t) if t is not None else None for t in ts]
    return L.attn_bwd_ex(ctypes.byref(pr or prob()), *r[:4], lse, *r[4:], ws, wsb, passes, None)


def test_ex_validation(L):
    assert L.attn_fwd_ex(None, *[ctypes.byref(T())] * 4, P, None) == 1
    for i in range(4):
        ts = [T() for _ in range(4)]
        ts[i] = None
        assert fwd_ex(L, ts=ts) == 1
        ts[i] = T(data=None)
        assert fwd_ex(L, ts=ts) == 1
        ts[i] = T(sn=-64)
        assert fwd_ex(L, ts=ts) == 10
        ts[i] = T(sn=60)
        assert fwd_ex(L, ts=ts) == 6
        ts[i] = T(sh=1 << 10 | 4)
        assert fwd_ex(L, ts=ts) == 6
        ts[i] = T(data=P + 8)
        assert fwd_ex(L, ts=ts) == 6
    assert fwd_ex(L, lse=None) == 1
    assert fwd_ex(L, lse=P + 4) == 6
    assert fwd_ex(L, pr=prob(dtype=2)) == 11
    assert fwd_ex(L, pr=prob(dtype=-1)) == 11
    assert fwd_ex(L, pr=prob(mask=3)) == 9
    assert fwd_ex(L, pr=prob(mask=ea.MASK_CAUSAL, window=4)) == 9
    assert fwd_ex(L, pr=prob(mask=ea.MASK_SLIDING_WINDOW, window=0)) == 9
    assert fwd_ex(L, pr=prob(d=112)) == 4
    assert fwd_ex(L, pr=prob(Hq=3, Hkv=2)) == 3
    assert fwd_ex(L, pr=prob(scale=0.0)) == 5
    assert fwd_ex(L, pr=prob(N=0)) == 2
    # shape errors win over stride errors, which win over alignment
    assert fwd_ex(L, pr=prob(N=0), ts=[T(sn=-8)] * 4) == 2
    assert fwd_ex(L, ts=[T(sn=-8), T(data=P + 2), T(), T()]) == 10


def test_bwd_ex_validation(L):
    assert bwd_ex(L, passes=0) == 12
    assert bwd_ex(L, passes=8) == 12
    assert bwd_ex(L, passes=15) == 12
    # order: dout, o (pre), q, k, v (main), dq, dk, dv; unused tensors may be NULL
    names = ["q", "k", "v", "o", "dout", "dq", "dk", "dv"]
    uses = {1: {"o", "dout"}, 2: {"q", "k", "v", "dout", "dk", "dv"}, 4: {"q", "k", "v", "dout", "dq"}}
    for bits, used in uses.items():
        for i, n in enumerate(names):
            ts = [T() for _ in range(8)]
            ts[i] = None
            r = bwd_ex(L, ts=ts, passes=bits, ws=None)
            assert r == (1 if n in used else 7), (bits, n, r)
            if n in used:
                ts[i] = T(sn=12)
                assert bwd_ex(L, ts=ts, passes=bits) == 6, (bits, n)
    assert bwd_ex(L, lse=None, passes=2) == 1
    assert bwd_ex(L, lse=None, passes=1, ws=None) == 1   # the preprocess rescales lse too
    assert bwd_ex(L, wsb=16) == 7
    assert bwd_ex(L, ws=P + 8) == 6
    assert bwd_ex(L, pr=prob(dtype=5)) == 11
    assert bwd_ex(L, pr=prob(mask=ea.MASK_NONE, window=3)) == 9
    assert bwd_ex(L, pr=prob(mask=ea.MASK_NONE, window=3), passes=1, ws=None) == 7  # no mask in pre
    assert bwd_ex(L, pr=prob(d=100)) == 4
    for bad in (1.0, -0.1, float("nan"), float("inf"), 2.0):
        assert bwd_ex(L, pr=prob(dropout_p=bad)) == 13
        assert bwd_ex(L, pr=prob(dropout_p=bad), passes=1, ws=None) == 7  # preprocess ignores it
        assert fwd_ex(L, pr=prob(dropout_p=bad)) == 13
    # the dropout check comes after shape / scale / mask / dtype
    assert fwd_ex(L, pr=prob(dropout_p=2.0, dtype=4)) == 11
    assert fwd_ex(L, pr=prob(dropout_p=0.5), lse=P + 4) == 6


def test_head_dims_have_plans(L):
    for d in ea.SUPPORTED_HEAD_DIMS:
        p = ea.fwd_plan(1, 4, 4, 1000, d)
        # two workgroups per CU, except one for d > 128 and for the
        # key-group plan (8 waves in two groups, twice the tile buffers)
        one_per_cu = d > 128 or p["key_groups"] == 2
        assert p["lds_bytes"] <= 160 * 1024 // (1 if one_per_cu else 2)
        assert p["block_kv"] == (64 if d <= 128 else 32)


# ------------------------------------------------------------------- decoding

def dprob(**kw):
    base = dict(B=2, Hq=8, Hkv=2, Nq=1, Nk=100, d=128, scale=0.1, mask=ea.MASK_CAUSAL, window=0,
                dtype=ea.DTYPE_BF16)
    base.update(kw)
    return ea.AttnDecodeProblem(*[base[f] for f, _ in ea.AttnDecodeProblem._fields_])


def dec(L, pr=None, ts=None, lens=None, lse=P, ws=P, wsb=1 << 24):
    ts = ts if ts is not None else [T() for _ in range(4)]
    r = [ctypes.byref(t) if t is not None else None for t in ts]
    return L.attn_decode_fwd(ctypes.byref(pr or dprob()), r[0], r[1], r[2], lens, r[3], lse, ws, wsb,
                             None)


def test_decode_validation(L):
    assert L.attn_decode_fwd(None, *[None] * 3, None, None, P, P, 1, None) == 1
    for i in range(4):
        ts = [T() for _ in range(4)]
        ts[i] = None
        assert dec(L, ts=ts) == 1
        ts[i] = T(sb=-8)
        assert dec(L, ts=ts) == 10
        ts[i] = T(sn=4)
        assert dec(L, ts=ts) == 6
    assert dec(L, lse=None) == 1
    assert dec(L, lse=P + 4) == 6
    assert dec(L, lens=P + 2) == 6
    assert dec(L, pr=dprob(Nq=0)) == 2
    assert dec(L, pr=dprob(Nk=0)) == 2
    assert dec(L, pr=dprob(Hq=6, Hkv=4)) == 3
    assert dec(L, pr=dprob(d=100)) == 4
    assert dec(L, pr=dprob(scale=-2.0)) == 5
    assert dec(L, pr=dprob(mask=ea.MASK_SLIDING_WINDOW, window=0)) == 9
    assert dec(L, pr=dprob(mask=ea.MASK_NONE, window=2)) == 9
    assert dec(L, pr=dprob(mask=7)) == 9
    assert dec(L, pr=dprob(dtype=3)) == 11
    need = L.attn_decode_workspace_bytes(ctypes.byref(dprob()))
    assert need > 0
    assert dec(L, ws=None) == 7
    assert dec(L, wsb=need - 1) == 7
    assert dec(L, ws=P + 8, wsb=need) == 6
    assert L.attn_decode_workspace_bytes(None) == 0
    assert L.attn_decode_workspace_bytes(ctypes.byref(dprob(d=100))) == 0
    # many sequences x KV heads fill the grid without splitting: no workspace
    assert L.attn_decode_workspace_bytes(ctypes.byref(dprob(B=4096, Hkv=8, Hq=8, Nk=64))) == 0


def test_decode_workspace_formula(L):
    # rows x splits x (d floats + 1 float), each part rounded up to 256 bytes
    pr = dprob(B=32, Hq=64, Hkv=8, Nq=1, Nk=4096, d=128)
    groups = 32 * 8
    S = -(-2048 // groups)
    LC = -(-4096 // S)
    LC = -(-LC // 32) * 32
    S = -(-4096 // LC)
    rows = 32 * 8 * 8
    want = -(-(rows * S * 128 * 4) // 256) * 256 + -(-(rows * S * 4) // 256) * 256
    assert L.attn_decode_workspace_bytes(ctypes.byref(pr)) == want


def noalloc(L, ptrs=None, B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125, causal=1):
    p = ptrs or [P] * 9
    return L.attn_bwd_noalloc(*p, B, Hq, Hkv, N, d, scale, causal, None)


def test_noalloc_validates_like_bwd(L):
    assert L.attn_bwd_noalloc_max_rows() == 1 << 21
    for which in range(9):
        ptrs = [P] * 9
        ptrs[which] = None
        assert noalloc(L, ptrs) == 1
    assert noalloc(L, N=0) == 2
    assert noalloc(L, Hq=3, Hkv=2) == 3
    assert noalloc(L, d=72) == 4
    assert noalloc(L, scale=0.0) == 5
    assert noalloc(L, ptrs=[P + 8] + [P] * 8) == 6


@pytest.mark.parametrize("B,Hq,N", [(1, 32, 65537), (4, 8, 65536 + 256), (1, 1, (1 << 21) + 1)])
def test_noalloc_rejects_problems_past_its_scratch(L, B, Hq, N):
    # more than 2^21 query rows: the fixed 16 MiB scratch cannot hold their row terms
    assert noalloc(L, B=B, Hq=Hq, Hkv=1, N=N) == 14


@pytest.mark.parametrize("probe", ["attn_probe_mfma_rate", "attn_probe_mfma16_rate"])
def test_mfma_probe_validates(L, probe):
    fn = getattr(L, probe)
    assert L.attn_probe_mfma_src_elems(3) == 3 * 512 * 16
    assert fn(None, P, 4, 8, 8, None) == 1
    assert fn(P, None, 4, 8, 8, None) == 1
    assert fn(P, P, 0, 8, 8, None) == 2
    assert fn(P, P, 4, 0, 8, None) == 2
    assert fn(P, P, (1 << 20) + 1, 8, 8, None) == 2
    assert fn(P, P, 4, 8, 3, None) == 2
