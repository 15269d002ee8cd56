"""The 32-key dK/dV kernel with each key block's query range split over two
workgroups, against the fp64 oracle (needs an MI355X).

On grids of at most one 128-key workgroup per CU (half that without a mask)
the heaviest key block's query loop decides the pass's time, so two
workgroups per key block each take half of its query blocks (the first one
the diagonal, masked blocks too) and write float32 partial dK and dV to the
workspace, which a second kernel adds in part order. These cases cover the
three masks, head dims 32 to 128, GQA (the part loops over the group's
heads), dropout, bf16 and fp16, BHSD and BSHD, and odd numbers of query
blocks per key block; each checks that its shape's workspace holds the
partials."""

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, N, d, mask, dtype, layout, dropout; B * Hkv * ceil(N / 128) <= 128
CASES = [
    (1, 2, 2, 4096, 128, "causal", "bf16", "bhsd", 0.0),
    (1, 4, 1, 1500, 64, "none", "fp16", "bshd", 0.0),
    (2, 4, 2, 2000, 80, 300, "bf16", "bhsd", 0.0),
    (1, 8, 8, 1030, 96, "causal", "bf16", "bhsd", 0.1),
    (1, 6, 3, 777, 32, "causal", "fp16", "bhsd", 0.0),
    (1, 16, 2, 1000, 128, "causal", "bf16", "bhsd", 0.0),
    (1, 2, 1, 600, 64, 1, "bf16", "bhsd", 0.0),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}_{}_{}_p{}".format(*c)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_query_split_dkdv(cfg):
    B, Hq, Hkv, N, d, mask, dt, layout, p = cfg
    parity.log(f"query-split dK/dV: {ids(cfg)}")
    row_terms = 2 * (-(-B * Hq * N * 4 // 256) * 256)
    assert ea.bwd_workspace_bytes(B, Hq, Hkv, N, d) == row_terms + 2 * 2 * B * Hkv * N * d * 4
    if mask == "none":
        kw, causal, window = dict(causal=False), False, None
    elif mask == "causal":
        kw, causal, window = dict(causal=True), True, None
    else:
        kw, causal, window = dict(window=mask), True, mask
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=9300 + N + d, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(d)
    p32 = float(np.float32(p))
    drop_kw = dict(dropout_p=p32, seed=0xA11 + N, offset=3) if p > 0 else {}
    drop = (p32, 0xA11 + N, 3) if p > 0 else None
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, layout=layout, **kw, **drop_kw)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, layout=layout, **kw, **drop_kw)
    torch.cuda.synchronize()
    if layout == "bshd":
        grads = tuple(t.transpose(1, 2) for t in grads)
    q, k, v, do = (si.to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, scale, causal, window=window, dropout=drop)
    for name, gg, r in (("dQ", grads[0], dQ), ("dK", grads[1], dK), ("dV", grads[2], dV)):
        e = parity.rel_l2(si.to_f64(gg), r)
        parity.log(f"  {name} rel L2 {e:.3e}")
        assert e <= parity.GRAD_TOL


def test_query_split_deterministic_and_passes_equal_fused():
    B, Hq, Hkv, N, d = 1, 4, 2, 2000, 64
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=4242, with_do=True)
    g = parity.to_gpu(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    a = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True)
    b = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True)
    dq, dk, dv = (torch.empty_like(t) for t in (g["q"], g["k"], g["v"]))
    ws = torch.empty(ea.bwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    for name in ("pre", "dkdv", "dq"):
        ea.bwd_passes(g["q"], g["k"], g["v"], o, lse, g["do"], dq, dk, dv, ws, causal=True, passes=(name,))
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, (dq, dk, dv)):
        assert torch.equal(x, y) and torch.equal(x, z)
