"""Sliding-window mask (keys i-W < j <= i) on the HIP path vs the fp64 oracle
(needs an MI355X). The band is the mask mode the CANN FlashAttention page lists
for long texts in its tuning section; the cases put its edges on, just before
and just after the forward's and backward's tile boundaries (32-row waves,
64/32-key forward steps, 128-key backward blocks), with ragged lengths."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, N, d, W
    (1, 2, 1, 50, 64, 1),
    (1, 2, 2, 130, 128, 2),
    (1, 4, 2, 300, 64, 31),
    (1, 2, 1, 300, 80, 32),
    (1, 2, 2, 300, 128, 33),
    (2, 4, 1, 517, 128, 64),
    (1, 2, 2, 700, 64, 100),
    (1, 3, 3, 600, 256, 127),
    (1, 2, 1, 600, 128, 128),
    (1, 2, 2, 601, 80, 129),
    (1, 8, 2, 1000, 128, 256),
    (1, 2, 2, 1000, 256, 257),
    (1, 2, 1, 2100, 64, 1000),
    (1, 2, 2, 300, 128, 299),
    (1, 2, 2, 300, 64, 300),
    (1, 2, 2, 300, 128, 301),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_W{}".format(*c)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_window_fwd_bwd(cfg):
    B, Hq, Hkv, N, d, W = cfg
    parity.log(f"case {ids(cfg)}")
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=31 + N + d + W, with_do=True)
    g = parity.to_gpu(inp)
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, window=W)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    parity.check_fwd(inp, o, lse, scale, True, heads, ids(cfg), window=W)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, window=W)
    torch.cuda.synchronize()
    kv_heads = [(b, h) for b in range(B) for h in range(Hkv)]
    parity.check_bwd(inp, grads, scale, True, kv_heads, Hq, Hkv, ids(cfg), window=W)


@pytest.mark.parametrize("shape", [
    (1, 4, 2, 333, 128),   # key groups in the forward and dQ
    (1, 4, 2, 1000, 64),   # also the query split in dK/dV (ragged last block)
    (1, 64, 8, 1000, 80),  # one group, one part
])
def test_window_covering_the_sequence_is_the_causal_mask(shape):
    """A band of N or more keys allows every j <= i: outputs are bit-identical
    to the causal call, on every plan."""
    N = shape[3]
    inp = parity.to_gpu(si.make_inputs(*shape, seed=41, with_do=True))
    o_c, l_c = ea.fwd(inp["q"], inp["k"], inp["v"], causal=True)
    g_c = ea.bwd(inp["q"], inp["k"], inp["v"], o_c, l_c, inp["do"], causal=True)
    for W in (N, N + 1, 1 << 20):
        o_w, l_w = ea.fwd(inp["q"], inp["k"], inp["v"], window=W)
        g_w = ea.bwd(inp["q"], inp["k"], inp["v"], o_w, l_w, inp["do"], window=W)
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_w) and torch.equal(l_c, l_w)
        for a, b in zip(g_c, g_w):
            assert torch.equal(a, b)


def test_window_of_one_key_copies_v():
    """With W = 1 each query sees only its own key: O_i = V_i exactly and
    LSE_i = scale * <q_i, k_i> (GQA: the KV head of the query head)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 64
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=43)
    g = parity.to_gpu(inp)
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, window=1)
    torch.cuda.synchronize()
    G = Hq // Hkv
    v_rep = inp["v"].repeat_interleave(G, dim=1)
    k_rep = inp["k"].double().repeat_interleave(G, dim=1)
    assert torch.equal(o.cpu(), v_rep)
    want = scale * (inp["q"].double() * k_rep).sum(-1)
    err = (lse.cpu().double() - want).abs().max().item()
    parity.log(f"[W=1] LSE max abs err {err:.3e}")
    assert err <= parity.LSE_TOL


def test_window_separate_passes_match_fused_call():
    inp = parity.to_gpu(si.make_inputs(1, 6, 3, 450, 128, seed=45, with_do=True))
    o, lse = ea.fwd(inp["q"], inp["k"], inp["v"], window=70)
    ref = ea.bwd(inp["q"], inp["k"], inp["v"], o, lse, inp["do"], window=70)
    outs = [torch.full_like(t, float("nan")) for t in ref]
    ws = torch.empty(ea.bwd_workspace_bytes(1, 6, 3, 450, 128), dtype=torch.uint8, device="cuda")
    ea.bwd_passes(inp["q"], inp["k"], inp["v"], o, lse, inp["do"], *outs, ws, window=70)
    torch.cuda.synchronize()
    for a, b in zip(ref, outs):
        assert torch.equal(a, b)
