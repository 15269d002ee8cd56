"""HIP path vs the fp64 oracle on seeded inputs (needs an MI355X).

Small shapes run through every head dimension (32, 64, 80, 96, 128, 192,
256), both mask modes, ragged lengths (not multiples of the tiles) and GQA
group sizes 1, 2, 3, 4, 8 and Hq.
Full workload shapes are checked on sampled heads (and, for the backward,
sampled KV-head groups), which the oracle computes exactly."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

SMALL = [
    # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 1, 17, 64, True),
    (2, 4, 2, 63, 80, False),
    (1, 4, 4, 64, 128, True),
    (1, 2, 2, 65, 256, True),
    (1, 8, 1, 129, 128, False),
    (1, 8, 8, 400, 64, False),
    (2, 8, 1, 1000, 80, True),
    (1, 16, 2, 1000, 128, True),
    (1, 3, 3, 257, 256, False),
    (1, 4, 2, 200, 256, True),
    (1, 2, 1, 300, 64, True),
    (1, 2, 2, 333, 80, True),
    (1, 2, 2, 190, 128, False),
    (1, 4, 2, 200, 32, True),
    (2, 2, 1, 97, 32, False),
    (1, 4, 1, 300, 96, True),
    (1, 2, 2, 130, 96, False),
    (1, 2, 1, 260, 192, True),
    (1, 2, 2, 70, 192, False),
    # past 512 keys: the step-loop forward at the head dims whose short
    # shapes take the key-split forward
    (1, 2, 1, 777, 32, True),
    (1, 2, 1, 700, 96, False),
    (1, 2, 2, 600, 64, False),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(*c[:5], "causal" if c[5] else "full")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", SMALL, ids=ids)
def test_small_fwd_bwd(cfg):
    B, Hq, Hkv, N, d, causal = cfg
    parity.log(f"case {ids(cfg)}")
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=7 + N + d, with_do=True)
    g = parity.to_gpu(inp)
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    parity.check_fwd(inp, o, lse, scale, causal, heads, ids(cfg))
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    kv_heads = [(b, h) for b in range(B) for h in range(Hkv)]
    parity.check_bwd(inp, grads, scale, causal, kv_heads, Hq, Hkv, ids(cfg))


def test_scale_argument_is_honoured():
    inp = si.make_inputs(1, 2, 1, 150, 64, seed=3, with_do=True)
    g = parity.to_gpu(inp)
    for scale in (0.02, 0.3):
        o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, causal=True)
        torch.cuda.synchronize()
        parity.check_fwd(inp, o, lse, scale, True, [(0, 0), (0, 1)], f"scale={scale}")
        grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, causal=True)
        torch.cuda.synchronize()
        parity.check_bwd(inp, grads, scale, True, [(0, 0)], 2, 1, f"scale={scale}")


def test_deterministic():
    inp = parity.to_gpu(si.make_inputs(1, 8, 2, 700, 128, seed=11, with_do=True))
    outs = []
    for _ in range(2):
        o, lse = ea.fwd(inp["q"], inp["k"], inp["v"], causal=True)
        dq, dk, dv = ea.bwd(inp["q"], inp["k"], inp["v"], o, lse, inp["do"], causal=True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_errors_raise_through_binding():
    q = torch.zeros((1, 2, 8, 112), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ea.AttnError) as e:
        ea.fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous())
    assert e.value.name == "ATTN_ERR_HEAD_DIM"
    q = torch.zeros((1, 3, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ea.AttnError) as e:
        ea.fwd(q, k, k)
    assert e.value.name == "ATTN_ERR_GQA"


def test_outputs_fully_overwritten():
    inp = parity.to_gpu(si.make_inputs(1, 2, 2, 77, 80, seed=5, with_do=True))
    o1, l1 = ea.fwd(inp["q"], inp["k"], inp["v"], causal=True)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    ea.fwd(inp["q"], inp["k"], inp["v"], causal=True, out=o2, lse=l2)
    g1 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], causal=True)
    gn = [torch.full_like(t, float("nan")) for t in g1]
    ws = torch.full((ea.bwd_workspace_bytes(1, 2, 2, 77, 80),), 255, dtype=torch.uint8, device="cuda")
    ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], causal=True, workspace=ws,
           dq=gn[0], dk=gn[1], dv=gn[2])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, gn):
        assert torch.equal(a, b)


def test_separate_passes_match_fused_call():
    inp = parity.to_gpu(si.make_inputs(2, 6, 3, 333, 128, seed=21, with_do=True))
    for causal in (False, True):
        o, lse = ea.fwd(inp["q"], inp["k"], inp["v"], causal=causal)
        ref = ea.bwd(inp["q"], inp["k"], inp["v"], o, lse, inp["do"], causal=causal)
        outs = [torch.full_like(t, float("nan")) for t in ref]
        ws = torch.empty(ea.bwd_workspace_bytes(2, 6, 3, 333, 128), dtype=torch.uint8, device="cuda")
        ea.bwd_passes(inp["q"], inp["k"], inp["v"], o, lse, inp["do"], *outs, ws, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b)
