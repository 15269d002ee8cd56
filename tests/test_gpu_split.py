"""The key-split forward for short sequences against the fp64 oracle (needs an
MI355X).

Shapes with at most 512 keys, head dims up to 96 and a grid of fewer than 256
workgroups of 128 rows run a kernel whose workgroup owns one 32-row query
tile and splits its keys over 2, 4 or 8 waves (64 keys each); the waves'
partial results are combined with the online-softmax rescaling identity.
These cases put N on, just below and just above the 32-row and 64-key tile
edges and the wave-count thresholds, cover all three masks, bf16 and fp16,
BHSD and BSHD views, and GQA, and check that each shape really takes that
plan. The backward runs on the split forward's LSE, so it is checked too."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, N, d, mask, dtype, layout
    (1, 2, 1, 1, 64, "causal", "bf16", "bhsd"),
    (1, 2, 2, 31, 32, "none", "bf16", "bhsd"),
    (1, 2, 1, 33, 64, "causal", "fp16", "bhsd"),
    (2, 4, 2, 63, 80, "none", "bf16", "bshd"),
    (1, 2, 2, 64, 96, "causal", "bf16", "bhsd"),
    (1, 4, 1, 65, 64, 7, "bf16", "bhsd"),
    (1, 2, 2, 127, 32, "causal", "fp16", "bshd"),
    (1, 3, 3, 128, 80, 40, "bf16", "bhsd"),
    (1, 2, 1, 129, 64, "none", "bf16", "bhsd"),
    (1, 8, 8, 200, 96, "none", "fp16", "bhsd"),
    (1, 2, 2, 255, 64, "causal", "bf16", "bhsd"),
    (1, 4, 2, 256, 80, 100, "bf16", "bshd"),
    (1, 2, 1, 257, 32, "none", "bf16", "bhsd"),
    (1, 8, 8, 400, 64, "none", "bf16", "bhsd"),
    (1, 8, 8, 400, 64, "causal", "bf16", "bhsd"),
    (2, 4, 4, 450, 96, 64, "fp16", "bhsd"),
    (1, 2, 2, 511, 80, "causal", "bf16", "bhsd"),
    (1, 6, 2, 512, 64, "none", "fp16", "bshd"),
    (1, 2, 1, 512, 32, 512, "bf16", "bhsd"),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}_{}_{}".format(*c)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_key_split_forward(cfg):
    B, Hq, Hkv, N, d, mask, dt, layout = cfg
    parity.log(f"split case {ids(cfg)}")
    if mask == "none":
        kw, causal, window = dict(causal=False), False, None
    elif mask == "causal":
        kw, causal, window = dict(causal=True), True, None
    else:
        kw, causal, window = dict(window=mask), True, mask
    plan = ea.fwd_plan(B, Hq, Hkv, N, d, causal)
    assert plan["key_splits"] > 1 and plan["block_q"] == 32, plan
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=5300 + N + d, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, layout=layout, **kw)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, layout=layout, **kw)
    torch.cuda.synchronize()
    if layout == "bshd":
        o = o.transpose(1, 2)
        grads = tuple(t.transpose(1, 2) for t in grads)
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    parity.check_fwd(inp, o, lse, scale, causal, heads, ids(cfg), window=window)
    kv_heads = [(b, h) for b in range(B) for h in range(Hkv)]
    parity.check_bwd(inp, grads, scale, causal, kv_heads, Hq, Hkv, ids(cfg), window=window)


def test_key_split_is_deterministic():
    inp = si.make_inputs(1, 8, 8, 400, 64, seed=1001)
    g = parity.to_gpu(inp)
    a = ea.fwd(g["q"], g["k"], g["v"])
    b = ea.fwd(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
