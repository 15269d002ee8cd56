"""attention(), the autograd form of the binding (needs an MI355X).

Its forward is fwd() and its backward bwd() on the saved q, k, v, O and LSE,
so its outputs and gradients must equal theirs bit for bit, in both layouts,
with GQA, windows and dropout (the backward redraws the forward's keep mask
from the same seed); and its gradients agree with the fp64 oracle."""

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


CASES = [
    # B, Hq, Hkv, N, d, layout, kwargs
    (1, 4, 2, 700, 64, "bhsd", dict(causal=True)),
    (2, 6, 3, 333, 128, "bshd", dict(causal=False)),
    (1, 4, 1, 1000, 80, "bhsd", dict(window=129)),
    (1, 2, 2, 600, 64, "bshd", dict(causal=True, dropout_p=0.125, seed=77, offset=5)),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(*c[:6]))
def test_attention_equals_fwd_bwd(cfg):
    B, Hq, Hkv, N, d, layout, kw = cfg
    parity.log(f"autograd {cfg}")
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=6100 + N, with_do=True)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    q, k, v = (g[x].detach().clone().requires_grad_(True) for x in ("q", "k", "v"))
    o = ea.attention(q, k, v, layout=layout, **kw)
    o.backward(g["do"])
    o_ref, lse = ea.fwd(g["q"], g["k"], g["v"], layout=layout, **kw)
    dq, dk, dv = ea.bwd(g["q"], g["k"], g["v"], o_ref, lse, g["do"], layout=layout, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for got, want in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert torch.equal(got, want)


def test_attention_drawn_seed_repeats_and_broadcast_grad():
    inp = si.make_inputs(1, 2, 2, 300, 64, seed=6200)
    g = parity.to_gpu(inp)
    outs = []
    for _ in range(2):
        torch.manual_seed(1234)
        q, k, v = (g[x].detach().clone().requires_grad_(True) for x in ("q", "k", "v"))
        o = ea.attention(q, k, v, causal=True, dropout_p=0.2)
        o.float().sum().backward()  # a broadcast (stride-0) gradient reaches the backward
        outs.append((o.detach(), q.grad, k.grad, v.grad))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.isfinite(a.float()).all() and torch.equal(a, b)


def test_attention_gradients_match_oracle():
    B, Hq, Hkv, N, d = 1, 4, 2, 520, 128
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=6300, with_do=True)
    g = parity.to_gpu(inp)
    q, k, v = (g[x].detach().clone().requires_grad_(True) for x in ("q", "k", "v"))
    o = ea.attention(q, k, v, causal=True)
    o.backward(g["do"])
    torch.cuda.synchronize()
    scale = ea.default_scale(d)
    qq, kk, vv, do = (si.to_f64(inp[x]) for x in ("q", "k", "v", "do"))
    dQ, dK, dV = oracle.ref_bwd(qq, kk, vv, do, scale, True)
    for name, got, ref in (("dQ", q.grad, dQ), ("dK", k.grad, dK), ("dV", v.grad, dV)):
        e = parity.rel_l2(si.to_f64(got), ref)
        parity.log(f"  {name} rel L2 {e:.3e}")
        assert e <= parity.GRAD_TOL
