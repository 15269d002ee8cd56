"""fp16 operands and strided layouts on the HIP path (needs an MI355X).

The CANN FlashAttention page (tuning section on data types) names float16
next to bfloat16; the yunthe.com GQA page calls flash_attn_func on
[batch, seq, heads, dim] tensors. fp16 results are checked against the fp64
oracle on the fp16 input values; layouts are checked for bit-identity with
the contiguous [B, H, N, d] call (same kernels, only the addressing
differs) and for leaving memory outside the output views untouched."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

FP16_CASES = [
    # B, Hq, Hkv, N, d, mask (None | "causal" | window)
    (1, 2, 1, 77, 64, None),
    (2, 4, 2, 300, 128, "causal"),
    (1, 4, 4, 129, 80, "causal"),
    (1, 2, 1, 500, 128, 100),
    (1, 2, 2, 200, 256, "causal"),
    (1, 4, 2, 150, 32, None),
    (1, 2, 1, 190, 96, "causal"),
    (1, 2, 2, 90, 192, 40),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_N{}_d{}_{}".format(*c[:5], c[5] if c[5] is not None else "full")


def mask_kw(m):
    if m is None:
        return dict(causal=False), False, None
    if m == "causal":
        return dict(causal=True), True, None
    return dict(window=m), True, m


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("cfg", FP16_CASES, ids=ids)
def test_fp16_matches_oracle(cfg):
    B, Hq, Hkv, N, d, m = cfg
    kw, causal, window = mask_kw(m)
    parity.log(f"fp16 case {ids(cfg)}")
    inp = si.make_inputs(B, Hq, Hkv, N, d, seed=51 + N + d, with_do=True, dtype="fp16")
    g = parity.to_gpu(inp)
    o, lse = ea.fwd(g["q"], g["k"], g["v"], **kw)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    scale = ea.default_scale(d)
    parity.check_fwd(inp, o, lse, scale, causal, [(b, h) for b in range(B) for h in range(Hq)],
                     "fp16 " + ids(cfg), window=window)
    grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], **kw)
    torch.cuda.synchronize()
    assert all(t.dtype == torch.float16 for t in grads)
    parity.check_bwd(inp, grads, scale, causal, [(b, h) for b in range(B) for h in range(Hkv)], Hq, Hkv,
                     "fp16 " + ids(cfg), window=window)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("m", [None, "causal", 64])
def test_bshd_is_bit_identical_to_bhsd(dtype, m):
    kw, _, _ = mask_kw(m)
    inp = parity.to_gpu(si.make_inputs(2, 6, 3, 333, 128, seed=61, with_do=True, dtype=dtype))
    o1, l1 = ea.fwd(inp["q"], inp["k"], inp["v"], **kw)
    g1 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], **kw)
    s = {key: si.in_layout(t, "bshd") for key, t in inp.items()}
    o2, l2 = ea.fwd(s["q"], s["k"], s["v"], layout="bshd", **kw)
    g2 = ea.bwd(s["q"], s["k"], s["v"], o2, l2, s["do"], layout="bshd", **kw)
    torch.cuda.synchronize()
    assert o2.shape == (2, 333, 6, 128) and o2.is_contiguous()
    assert torch.equal(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert b.is_contiguous()
        assert torch.equal(a, b.transpose(1, 2))


def test_packed_qkv_views_and_guarded_outputs():
    """q, k, v as views into one packed [B, N, 3, H, d] buffer (d contiguous,
    other strides arbitrary multiples of 8), outputs written into the middle
    of larger buffers whose other elements must keep their guard values."""
    B, H, N, d = 2, 4, 257, 64
    inp = si.make_inputs(B, H, H, N, d, seed=71, with_do=True)
    packed = torch.stack([si.in_layout(inp[x], "bshd") for x in ("q", "k", "v")], dim=2).cuda()
    q, k, v = (packed[:, :, i].transpose(1, 2) for i in range(3))  # [B, H, N, d] views
    assert not q.is_contiguous()
    do = inp["do"].cuda()
    big_o = torch.full((B, H, N + 3, d + 16), 7.0, dtype=torch.bfloat16, device="cuda")
    o_view = big_o[:, :, 2:N + 2, 8:8 + d]
    o, lse = ea.fwd(q, k, v, causal=True, out=o_view)
    big_g = [torch.full((B, H, N + 1, d + 8), -3.0, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    gv = [t[:, :, 1:, 8:] for t in big_g]
    ea.bwd(q, k, v, o, lse, do, causal=True, dq=gv[0], dk=gv[1], dv=gv[2])
    ref_o, ref_l = ea.fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal=True)
    ref_g = ea.bwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), ref_o, ref_l, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_view, ref_o) and torch.equal(lse, ref_l)
    mask = torch.ones_like(big_o, dtype=torch.bool)
    mask[:, :, 2:N + 2, 8:8 + d] = False
    assert bool((big_o[mask] == 7.0).all())
    for t, view, ref in zip(big_g, gv, ref_g):
        assert torch.equal(view, ref)
        m = torch.ones_like(t, dtype=torch.bool)
        m[:, :, 1:, 8:] = False
        assert bool((t[m] == -3.0).all())


@pytest.mark.parametrize("m", [None, "causal", 50])
def test_strided_entry_point_matches_plain_one(m):
    """attn_fwd_ex / attn_bwd_ex on contiguous bf16 tensors give the plain
    entry points' results bit for bit."""
    kw, _, _ = mask_kw(m)
    inp = parity.to_gpu(si.make_inputs(1, 4, 2, 300, 80, seed=81, with_do=True))
    o1, l1 = ea.fwd(inp["q"], inp["k"], inp["v"], **kw)
    o2, l2 = ea.fwd(inp["q"], inp["k"], inp["v"], use_ex=True, **kw)
    g1 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], **kw)
    g2 = ea.bwd(inp["q"], inp["k"], inp["v"], o1, l1, inp["do"], use_ex=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dtype_errors():
    q = torch.zeros((1, 2, 8, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        ea.fwd(q, q, q)
    a = torch.zeros((1, 2, 8, 64), dtype=torch.float16, device="cuda")
    b = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        ea.fwd(a, b, b)
