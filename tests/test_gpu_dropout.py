"""Fused dropout on the HIP path vs the fp64 oracle (needs an MI355X).

The CANN FlashAttention page (tuning section) asks for dropout inside the
fused kernel during training. Both sides draw the keep mask from the same
counter-based stream (Philox-4x32-10, written independently in
oracle/philox.py and in the kernels), so the masks must agree bit for bit
and the outputs to the usual tolerances."""

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from oracle import philox
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, N, d, mask, p, dtype
    (1, 2, 1, 100, 64, "causal", 0.1, "bf16"),
    (2, 4, 2, 257, 128, "none", 0.3, "bf16"),
    (1, 4, 4, 130, 80, "causal", 0.5, "bf16"),
    (1, 2, 1, 300, 128, 70, 0.2, "bf16"),
    (1, 2, 2, 129, 256, "causal", 0.15, "bf16"),
    (1, 4, 2, 200, 32, "none", 0.4, "fp16"),
    (1, 2, 1, 190, 96, "causal", 0.25, "fp16"),
    (1, 2, 2, 97, 192, "causal", 0.1, "bf16"),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}_p{}_{}".format(*c)


def mask_kw(m):
    if m == "none":
        return dict(causal=False), False, None
    if m == "causal":
        return dict(causal=True), True, None
    return dict(window=m), True, m


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_dropout_matches_oracle(cfg):
    B, Hq, Hkv, N, d, m, p, dt = cfg
    parity.log(f"dropout case {ids(cfg)}")
    kw, causal, window = mask_kw(m)
    seed, offset = 0x1234_5678_9ABC + N, 17 + d
    p32 = float(np.float32(p))
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=101 + N + d, with_do=True, dtype=dt)
    g = parity.to_gpu(inp)
    scale = ea.default_scale(d)
    dk = dict(dropout_p=p32, seed=seed, offset=offset)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, **kw, **dk)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, **kw, **dk)
    torch.cuda.synchronize()
    q, k, v, do = (si.to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    drop = (p32, seed, offset)
    O, L = oracle.ref_fwd(q, k, v, scale, causal, window=window, dropout=drop)
    # Kept weights are scaled by 1/(1-p), so |O| can leave the range of V and
    # the 16-bit rounding of O (half an ulp: 2^-8 |O| for bf16, 2^-11 for
    # fp16) is added to the absolute bound.
    rel = 2.0 ** -8 if dt == "bf16" else 2.0 ** -11
    err = np.abs(si.to_f64(o) - O)
    eo = float(err.max())
    el = float(np.abs(lse.cpu().double().numpy() - L).max())
    parity.log(f"[dropout fwd {ids(cfg)}] O {eo:.3e} (max |O| {np.abs(O).max():.2f}) LSE {el:.3e}")
    assert np.all(err <= parity.O_TOL + rel * np.abs(O)) and el <= parity.LSE_TOL
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, scale, causal, window=window, dropout=drop)
    for name, gg, r in (("dQ", grads[0], dQ), ("dK", grads[1], dK), ("dV", grads[2], dV)):
        e = parity.rel_l2(si.to_f64(gg), r)
        parity.log(f"[dropout bwd {ids(cfg)}] {name} rel L2 {e:.3e}")
        assert e <= parity.GRAD_TOL


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_dropout_mask_is_bit_exact(dt):
    """With V = identity rows (N = d) O_ij = P_ij M_ij / (1 - p): the zero
    pattern of O is the kernel's keep mask, compared with the oracle's."""
    B, H, N, d, p = 2, 3, 128, 128, 0.37
    p32 = float(np.float32(p))
    inp = si.make_inputs(B, H, H, N, d, seed=103, dtype=dt)
    v = torch.eye(N, dtype=inp["v"].dtype).expand(B, H, N, d).contiguous()
    q = (inp["q"].float() * 0.1).to(inp["q"].dtype)  # keep every weight well above zero
    o, _ = ea.fwd(q.cuda(), inp["k"].cuda(), v.cuda(), causal=False, dropout_p=p32, seed=77, offset=5)
    torch.cuda.synchronize()
    got = (o.float().cpu().numpy() != 0)
    for b in range(B):
        for h in range(H):
            want = philox.dropout_keep(b * H + h, np.arange(N), np.arange(N), p32, 77, 5)
            assert np.array_equal(got[b, h], want), f"mask differs for head {(b, h)}"
    frac = got.mean()
    parity.log(f"[dropout mask {dt}] kept fraction {frac:.4f} (1 - p = {1 - p:.4f})")


def test_dropout_streams_and_determinism():
    inp = parity.to_gpu(si.make_inputs(1, 4, 2, 200, 64, seed=105, with_do=True))
    kw = dict(causal=True, dropout_p=0.25)
    o1, l1 = ea.fwd(inp["q"], inp["k"], inp["v"], seed=1, offset=0, **kw)
    o2, l2 = ea.fwd(inp["q"], inp["k"], inp["v"], seed=1, offset=0, **kw)
    o3, l3 = ea.fwd(inp["q"], inp["k"], inp["v"], seed=1, offset=1, **kw)
    o4, _ = ea.fwd(inp["q"], inp["k"], inp["v"], seed=2, offset=0, **kw)
    g1 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], seed=1, offset=0, **kw)
    g2 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], seed=1, offset=0, **kw)
    o0, l0 = ea.fwd(inp["q"], inp["k"], inp["v"], causal=True)
    oz, lz = ea.fwd(inp["q"], inp["k"], inp["v"], causal=True, use_ex=True, dropout_p=0.0, seed=9)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert not torch.equal(o1, o3) and not torch.equal(o1, o4)
    # dropout leaves the LSE alone: bit for bit between dropout streams (one
    # kernel), and to fp32 rounding against the plain forward, which takes
    # the key-split plan at this length and so sums in another order
    assert torch.equal(l1, l3)
    assert float((l1 - l0).abs().max()) <= 1e-5
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    assert torch.equal(o0, oz) and torch.equal(l0, lz)
