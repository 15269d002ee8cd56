"""Parity at the full workload shapes, on sampled heads, in the launch
configuration the bench times (needs an MI355X)."""

import pytest
import torch

import exact_attention_12_amd as ea
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

FWD_HEADS = {
    "c1_yolo_n400": None,  # all heads
    "c2_mha_n512": [(0, 0), (3, 15)],
    "c2_mha_n1024": [(0, 0), (3, 15)],
    "c2_mha_n2048": [(1, 7), (3, 15)],
    "c2_mha_n4096": [(0, 0), (3, 15)],
    "c3_causal_7b": [(0, 0), (1, 31)],
    "c4_gqa_70b": [(0, 0), (0, 9), (0, 63)],
    "c4_mqa_70b": [(0, 0), (0, 63)],
    "c4_gqa_70b_bwd": [(0, 5), (0, 60)],
    "c5_bwd_d128": [(0, 0), (0, 15)],
    "c5_bwd_d80": [(0, 0), (0, 5), (0, 15)],
    "c6_window_d128": [(0, 0), (0, 31)],
    "c7_fp16_bshd_d128": [(0, 0), (0, 15)],
    "c9_dropout_d128": [(0, 2), (0, 15)],
}
BWD_KV_HEADS = {
    "c4_gqa_70b_bwd": [(0, 3)],
    "c5_bwd_d128": [(0, 3)],
    "c5_bwd_d80": [(0, 0), (0, 15)],
    "c6_window_d128": [(0, 5)],
    "c7_fp16_bshd_d128": [(0, 7)],
    "c9_dropout_d128": [(0, 11)],
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.lib()


@pytest.mark.parametrize("name", list(FWD_HEADS))
def test_workload(name):
    w = si.WORKLOADS[name]
    parity.log(f"workload {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.mask} "
               f"{w.dtype} {w.layout}")
    inp = si.workload_inputs(w)
    g = {key: si.in_layout(t.cuda(), w.layout) for key, t in inp.items()}
    dk = {} if w.dropout is None else dict(dropout_p=w.dropout[0], seed=w.dropout[1], offset=w.dropout[2])
    o, lse = ea.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, window=w.window,
                    layout=w.layout, **dk)
    torch.cuda.synchronize()
    if w.layout == "bshd":  # back to [B, H, N, d] for the checks
        o = o.transpose(1, 2)
        g = {key: t.transpose(1, 2) for key, t in g.items()}
    heads = FWD_HEADS[name] or [(b, h) for b in range(w.B) for h in range(w.Hq)]
    parity.check_fwd(inp, o, lse, w.scale, w.causal, heads, name, window=w.window, dropout=w.dropout)
    if w.backward:
        grads = ea.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], scale=w.scale, causal=w.causal,
                       window=w.window, **dk)  # BHSD views of the same memory
        torch.cuda.synchronize()
        parity.check_bwd(inp, grads, w.scale, w.causal, BWD_KV_HEADS[name], w.Hq, w.Hkv, name,
                         window=w.window, dropout=w.dropout)
        # Identities that hold for every head: rows of P sum to one, so the
        # key-sum of dV equals the query-sum of dO over each group; shifting
        # all keys leaves O unchanged, so the key-sum of dK vanishes.
        dk, dv = grads[1].double(), grads[2].double()
        do_sum = g["do"].double().sum(dim=2).reshape(w.B, w.Hkv, w.G, w.d).sum(dim=2)
        rel = (dv.sum(dim=2) - do_sum).norm() / do_sum.norm()
        parity.log(f"[{name}] sum_j dV_j vs sum_i dO_i rel err {rel:.3e}")
        assert rel < parity.GRAD_TOL
        dk_sum = dk.sum(dim=2).norm() / (dk.norm() / (w.N ** 0.5) + 1e-30) / (w.N ** 0.5)
        parity.log(f"[{name}] |sum_j dK_j| relative to sqrt(N)*rms row {dk_sum:.3e}")
        assert dk_sum < 0.05
