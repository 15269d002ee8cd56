"""The d = 128 forward and dQ pass on 16x16x32 products against the fp64
oracle (needs an MI355X).

Without dropout, grids large enough for the 8-wave plan at other head dims
run the forward's step loop on 16x16x32 products (fwd_m16_kernel, 4 waves
per workgroup, two workgroups per CU): each wave holds two 16-query
tiles, its lanes hold 16 keys of a query in four 16-lane groups, and the
probabilities of a 32-key half are packed as the B operand in the key order
(4g .. 4g+3, 16+4g .. 16+4g+3) that the V^T operand is read in. The row
maximum and sum combine the four groups; the reference maximum is only
re-derived across the groups when some lane's own maximum could move it.
The dQ pass of these shapes (one key group: grids too large for key groups)
runs bwd_dq_m16_kernel, the same layout for S^T, dP^T and dQ^T += K^T dS^T,
with the K tile read both row-wise and transposed through a chunk swizzle.
These cases check that each shape takes that plan and cover the three masks
(a window of 1 leaves most of a wave's rows with no allowed key in its first
tiles), ragged N with a lone row in the last block, GQA and MQA, bf16 and
fp16, BHSD and BSHD; the backward runs on this forward's LSE and is checked
too. The rows whose running maximum moves again and again along the
sequence are covered on this plan by the rescale tests' m16 cases."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

D = 128
LDS_BYTES = 2 * 64 * (144 + 144) * 2  # two K and two V buffers, pitch 288 bytes

# B, Hq, Hkv, N, mask, dtype, layout
CASES = [
    (1, 128, 16, 1000, "causal", "bf16", "bhsd"),
    (2, 64, 8, 777, "none", "bf16", "bhsd"),
    (1, 128, 128, 1100, 300, "fp16", "bhsd"),
    (1, 128, 1, 1000, "causal", "fp16", "bhsd"),
    (1, 128, 32, 1025, 40, "bf16", "bshd"),
    (2, 128, 64, 257, "causal", "bf16", "bhsd"),
    (1, 128, 16, 1030, 1, "bf16", "bhsd"),
    (1, 64, 64, 2049, "none", "fp16", "bshd"),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_{}_{}_{}".format(*c)


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


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_products16_forward(cfg):
    B, Hq, Hkv, N, mask, dt, layout = cfg
    parity.log(f"16x16x32 forward case {ids(cfg)}")
    kw, causal, window = mask_args(mask)
    plan = ea.fwd_plan(B, Hq, Hkv, N, D, causal)
    assert plan["key_splits"] == 1 and plan["key_groups"] == 1, plan
    assert plan["products16"] == 1 and plan["threads"] == 256 and plan["block_q"] == 128, plan
    assert plan["lds_bytes"] == LDS_BYTES, plan
    inp = si.make_inputs(B, Hq, Hkv, N, D, seed=8100 + N + Hkv, with_do=True, dtype=dt)
    g = {key: si.in_layout(t.cuda(), layout) for key, t in inp.items()}
    scale = ea.default_scale(D)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, layout=layout, **kw)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, layout=layout, **kw)
    torch.cuda.synchronize()
    if layout == "bshd":
        o = o.transpose(1, 2)
        grads = tuple(t.transpose(1, 2) for t in grads)
    # the first and last batch's first and last KV group, all of their query heads
    G = Hq // Hkv
    heads = sorted({(b, h) for b in (0, B - 1) for hk in (0, Hkv - 1) for h in range(hk * G, (hk + 1) * G)})
    heads = heads[:16] + heads[-16:] if len(heads) > 32 else heads
    parity.check_fwd(inp, o, lse, scale, causal, heads, ids(cfg), window=window)
    kv_heads = sorted({(b, h * Hkv // Hq) for b, h in heads})[:4]
    parity.check_bwd(inp, grads, scale, causal, kv_heads, Hq, Hkv, ids(cfg), window=window)


def test_products16_plan_only_on_large_grids():
    # the plans of smaller grids stay on the 32x32x16 kernel (its V pitch)
    p = ea.fwd_plan(1, 32, 32, 1000, D, True)
    assert p["threads"] == 256 and p["key_groups"] == 1 and p["products16"] == 0, p
    assert p["lds_bytes"] == 2 * 64 * ((D + 8) + 160) * 2, p


def test_products16_deterministic():
    inp = si.make_inputs(1, 128, 16, 1000, D, seed=8101)
    g = parity.to_gpu(inp)
    a = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    b = ea.fwd(g["q"], g["k"], g["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
