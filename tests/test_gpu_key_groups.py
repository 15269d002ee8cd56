"""The forward with two key groups per workgroup against the fp64 oracle
(needs an MI355X).

When the grid is small next to the longest query block's key loop, the
forward's 4 waves form two groups of 2 over one 64-row query block: group 0
walks the first half of the block's 64-key tiles, group 1 the rest (one tile
fewer when their number is odd, so group 1 idles through the last step), and
the two partial online-softmax states are combined in LDS. These cases check
that each shape takes that plan and cover all three masks (a window of 1
leaves many rows with no allowed key in group 0), every head dim up to 128,
ragged N, GQA and MQA, bf16 and fp16, BHSD and BSHD. The backward runs on
this forward's LSE, so it is checked too. A second set has the same kinds of
ragged shapes on grids large enough for the one-group kernel."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, N, d, mask, dtype, layout
GROUPED = [
    (1, 2, 1, 777, 32, "causal", "bf16", "bhsd"),
    (1, 2, 2, 601, 80, "causal", "fp16", "bshd"),
    (1, 4, 2, 1000, 64, "none", "bf16", "bhsd"),
    (1, 2, 2, 700, 96, 100, "bf16", "bhsd"),
    (1, 4, 4, 999, 128, "causal", "bf16", "bhsd"),
    (2, 4, 2, 300, 128, "none", "fp16", "bhsd"),
    (1, 8, 1, 517, 128, 1, "bf16", "bshd"),
    (1, 2, 1, 1500, 80, 300, "bf16", "bhsd"),
    (1, 2, 2, 257, 128, "causal", "bf16", "bhsd"),
    (1, 4, 2, 2100, 64, "causal", "bf16", "bhsd"),
    (2, 3, 1, 450, 128, 64, "fp16", "bhsd"),
]
ONE_GROUP = [
    (4, 32, 8, 1000, 128, "causal", "bf16", "bhsd"),
    (4, 32, 32, 777, 80, "none", "fp16", "bshd"),
    (16, 16, 4, 600, 64, 150, "bf16", "bhsd"),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}_{}_{}".format(*c)


def mask_args(mask):
    if mask == "none":
        return dict(causal=False), False, None
    if mask == "causal":
        return dict(causal=True), True, None
    return dict(window=mask), True, mask


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


def run_case(cfg, groups, check_heads=None):
    B, Hq, Hkv, N, d, mask, dt, layout = cfg
    parity.log(f"key-group case {ids(cfg)} (groups {groups})")
    kw, causal, window = mask_args(mask)
    plan = ea.fwd_plan(B, Hq, Hkv, N, d, causal)
    assert plan["key_splits"] == 1 and plan["key_groups"] == groups, plan
    if groups == 2:
        assert plan["block_q"] == 64 and plan["threads"] == 256, plan
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=5700 + N + d, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(d)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, layout=layout, **kw)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, layout=layout, **kw)
    torch.cuda.synchronize()
    if layout == "bshd":
        o = o.transpose(1, 2)
        grads = tuple(t.transpose(1, 2) for t in grads)
    heads = check_heads or [(b, h) for b in range(B) for h in range(Hq)]
    parity.check_fwd(inp, o, lse, scale, causal, heads, ids(cfg), window=window)
    kv_heads = sorted({(b, h * Hkv // Hq) for b, h in heads})
    parity.check_bwd(inp, grads, scale, causal, kv_heads, Hq, Hkv, ids(cfg), window=window)


@pytest.mark.parametrize("cfg", GROUPED, ids=ids)
def test_key_groups_forward(cfg):
    run_case(cfg, 2)


@pytest.mark.parametrize("cfg", ONE_GROUP, ids=ids)
def test_one_group_ragged(cfg):
    B, Hq, Hkv = cfg[:3]
    # the first and last batch's first KV group, all of its query heads
    G = Hq // Hkv
    heads = [(b, h) for b in (0, B - 1) for h in range(G)]
    run_case(cfg, 1, heads)


def test_key_groups_deterministic():
    inp = si.make_inputs(1, 4, 4, 999, 128, seed=1002)
    g = parity.to_gpu(inp)
    a = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    b = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
