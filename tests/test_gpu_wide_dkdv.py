"""The 64-keys-per-wave dK/dV kernel (d = 128), which the backward
uses once there are at least 512 blocks of 256 keys (B * Hkv * ceil(N / 256)),
or at least 256 of them with an even group size, splitting each group's
query heads over two workgroups.
The other GPU tests reach it only at the large workload shapes, through sampled
rows; these shapes are just above that size, ragged (N not a multiple of 256
or 32), so every element of dQ, dK and dV is checked against the fp64 oracle.
Together they cover causal, window and no mask, GQA, both element types,
both layouts and dropout."""

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, N, mask, dtype, layout, dropout; each has >= 512 blocks of 256 keys
CASES = [
    (2, 52, 52, 1285, "causal", "bf16", "bhsd", 0.0),   # 6 blocks x 104
    (1, 256, 128, 1037, 300, "bf16", "bhsd", 0.0),      # window, G = 2: 5 x 128
    (4, 32, 32, 1031, "none", "fp16", "bshd", 0.0),     # 5 x 128
    (1, 104, 104, 1285, "causal", "bf16", "bhsd", 0.2),  # 6 x 104
    (1, 128, 128, 1030, 300, "fp16", "bshd", 0.1),      # 5 x 128
    # 256 .. 511 blocks, G even: the query heads of a group split over two
    # workgroups, partial sums added by a second kernel
    (1, 256, 128, 520, "causal", "bf16", "bhsd", 0.0),  # 3 x 128
    (1, 128, 64, 1030, 300, "fp16", "bshd", 0.1),       # 5 x 64, window, dropout
    # dropout with two query heads per workgroup: each step's keep bits must
    # come from that step's head (G = 2 unsplit; G = 4 split in two)
    (1, 256, 128, 1037, "causal", "bf16", "bhsd", 0.1),  # 5 x 128
    (1, 128, 32, 1800, "causal", "fp16", "bshd", 0.1),   # 8 x 32, split
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_{}_{}_{}_p{}".format(*c)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_wide_dkdv(cfg):
    B, Hq, Hkv, N, mask, dt, layout, p = cfg
    d = 128
    n4 = B * Hkv * ((N + 255) // 256)
    assert n4 >= 512 or (2 * n4 >= 512 and (Hq // Hkv) % 2 == 0)
    parity.log(f"wide dK/dV: {ids(cfg)}")
    if mask == "none":
        kw, causal, window = dict(causal=False), False, None
    elif mask == "causal":
        kw, causal, window = dict(causal=True), True, None
    else:
        kw, causal, window = dict(window=mask), True, mask
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=9100 + N, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(d)
    p32 = float(np.float32(p))
    drop_kw = dict(dropout_p=p32, seed=0xD1CE + N, offset=5) if p > 0 else {}
    drop = (p32, 0xD1CE + N, 5) if p > 0 else None
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
