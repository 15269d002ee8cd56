"""attn_bwd_noalloc (the backward with the library's fixed scratch in place of
a caller's workspace) against attn_bwd, through the C ABI (needs an MI355X).

Two calls in a row share the one scratch array of the GPU, the second with a
smaller problem than the first, so a row term left over from the first call
would show in the second. Where both entry points run the same kernels the
results must agree bit for bit; on the grouped shape where attn_bwd sums two
fp32 halves of dK/dV in its workspace the no-allocation call runs a single
dK/dV pass, so dK and dV are compared to the oracle tolerance (and far
tighter) while dQ stays bit-identical. The first shape's gradients are also
checked against the fp64 oracle on a sampled KV-head group."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

CALLS = [
    # B, Hq, Hkv, N, d, causal, bitwise dK/dV (same dK/dV kernel as attn_bwd)
    (1, 16, 8, 8192, 128, True, False),   # attn_bwd splits the group's heads over two passes here
    (1, 4, 2, 1000, 64, True, True),
    (2, 4, 4, 777, 128, False, True),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


def test_noalloc_matches_bwd_on_consecutive_calls():
    for i, (B, Hq, Hkv, N, d, causal, bitwise) in enumerate(CALLS):
        parity.log(f"no-alloc call {i}: B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
        inp = si.make_inputs(B, Hq, Hkv, N, d, seed=4400 + i, with_do=True)
        g = parity.to_gpu(inp)
        scale = ea.default_scale(d)
        o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=scale, causal=causal)
        ref = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=scale, causal=causal)
        outs = tuple(torch.full_like(t, float("nan")) for t in ref)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        ea.bwd_noalloc(g["q"], g["k"], g["v"], o, lse, g["do"], *outs, scale=scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        for name, a, r in zip(("dQ", "dK", "dV"), outs, ref):
            assert torch.isfinite(a).all(), name
            if name == "dQ" or bitwise:
                assert torch.equal(a, r), f"{name} differs from attn_bwd"
            else:
                e = parity.rel_l2(si.to_f64(a), si.to_f64(r))
                parity.log(f"  {name} rel L2 vs attn_bwd {e:.2e}")
                assert e <= 1e-3
        if i == 0:
            parity.check_bwd(inp, outs, scale, causal, [(0, 3)], Hq, Hkv, "no-alloc")


def test_noalloc_limit():
    assert ea.bwd_noalloc_max_rows() == 1 << 21
