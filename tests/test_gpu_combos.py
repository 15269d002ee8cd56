"""Every combination of the features that can meet in one call, on small
ragged shapes, against the fp64 oracle (needs an MI355X): element type
(bf16, fp16) x layout (BHSD, BSHD views) x mask (none, causal, window of 37
keys) x dropout (off, p = 0.2), with a KV head shared by two query heads, at
d = 64 and d = 128 (the two tile paths of the forward and both backward
kernels). Each feature is tested in depth elsewhere; this catches their
interactions (strides with the dropout stream, fp16 with windows, ...)."""

import itertools

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

CASES = list(itertools.product(["bf16", "fp16"], ["bhsd", "bshd"], ["none", "causal", 37],
                               [0.0, 0.2], [64, 128]))


def ids(c):
    dt, layout, mask, p, d = c
    return f"{dt}_{layout}_{mask}_p{p}_d{d}"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_combination(cfg):
    dt, layout, mask, p, d = cfg
    B, Hq, Hkv, N = 2, 4, 2, 161
    parity.log(f"combination {ids(cfg)}")
    if mask == "none":
        kw, causal, window = dict(causal=False), False, None
    elif mask == "causal":
        kw, causal, window = dict(causal=True), True, None
    else:
        kw, causal, window = dict(window=mask), True, mask
    p32 = float(np.float32(p))
    drop_kw = dict(dropout_p=p32, seed=0xC0FFEE + d, offset=3) if p > 0 else {}
    drop = (p32, 0xC0FFEE + d, 3) if p > 0 else None

    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=7000 + d + N, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, layout=layout, **kw, **drop_kw)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, layout=layout, **kw, **drop_kw)
    torch.cuda.synchronize()
    if layout == "bshd":  # back to [B, H, N, d] views for the checks
        o = o.transpose(1, 2)
        grads = tuple(t.transpose(1, 2) for t in grads)

    q, k, v, do = (si.to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    O, L = oracle.ref_fwd(q, k, v, scale, causal, window=window, dropout=drop)
    # kept weights are scaled by 1/(1-p), so under dropout |O| can leave the
    # range of V: the 16-bit rounding of O (half an ulp) is added to the
    # absolute bound then, and only then
    rel = 0.0 if p == 0 else (2.0 ** -8 if dt == "bf16" else 2.0 ** -11)
    err = np.abs(si.to_f64(o) - O)
    el = float(np.abs(lse.cpu().double().numpy() - L).max())
    parity.log(f"  O {float(err.max()):.3e} LSE {el:.3e}")
    assert np.all(err <= parity.O_TOL + rel * np.abs(O)) and el <= parity.LSE_TOL
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, scale, causal, window=window, dropout=drop)
    for name, gg, r in (("dQ", grads[0], dQ), ("dK", grads[1], dK), ("dV", grads[2], dV)):
        e = parity.rel_l2(si.to_f64(gg), r)
        parity.log(f"  {name} rel L2 {e:.3e}")
        assert e <= parity.GRAD_TOL
