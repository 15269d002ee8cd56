"""Decoding against a KV cache on the HIP path vs the fp64 oracle (needs an
MI355X). The cache and its GQA sharing follow the yunthe.com GQA page
(sections on the MHA KV cache and on GQA); query i of sequence b is the
token at position L_b - Nq + i (see oracle.ref_decode)."""

import numpy as np
import pytest
import torch

import exact_attention_12_amd as ea
import oracle
import synthetic_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Nq, Nk, d, mask, lens ("full" | "ragged"), dtype
    (4, 8, 1, 1, 1000, 128, "causal", "full", "bf16"),
    (3, 16, 2, 1, 777, 64, "none", "ragged", "bf16"),
    (2, 8, 8, 4, 513, 80, "causal", "ragged", "bf16"),
    (2, 64, 1, 1, 300, 128, "causal", "full", "bf16"),   # G = 64: two row tiles
    (1, 8, 2, 16, 2000, 128, "causal", "full", "bf16"),  # R = 64
    (2, 4, 2, 3, 450, 256, 100, "ragged", "bf16"),
    (5, 4, 4, 2, 129, 32, "causal", "ragged", "fp16"),
    (2, 12, 4, 1, 333, 96, 64, "full", "fp16"),
    (64, 8, 8, 1, 256, 128, "causal", "ragged", "bf16"),  # many groups: one split
    (1, 32, 8, 1, 20000, 128, "causal", "full", "bf16"),  # long cache: many splits
    (1, 8, 1, 2, (1 << 20) + 77, 128, "causal", "full", "bf16"),  # 2^20 keys: 2048 splits
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_{}_{}".format(*c)


def lens_for(kind, B, Nk, Nq, seed):
    if kind == "full":
        return None
    r = np.random.default_rng(seed)
    lens = r.integers(1, Nk + 1, size=B)
    # edge cases: an empty cache, fewer rows than new queries, a length past
    # the cache (clamped), a full cache
    extra = [0, max(Nq - 1, 0), Nk + 5, Nk]
    for j, x in enumerate(extra[:B]):
        lens[j] = x
    return lens.astype(np.int32)


def mask_args(m):
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


def check(inp, lens, o, lse, scale, causal, window, tag):
    q, k, v = (si.to_f64(inp[x]) for x in ("q", "k", "v"))
    O, L = oracle.ref_decode(q, k, v, scale, causal, kv_lens=lens, window=window)
    og = si.to_f64(o)
    lg = lse.detach().cpu().double().numpy()
    assert np.isfinite(og).all()
    assert np.array_equal(np.isneginf(lg), np.isneginf(L)), "rows without keys differ"
    fin = np.isfinite(L)
    eo = float(np.abs(og - O).max())
    el = float(np.abs(lg[fin] - L[fin]).max()) if fin.any() else 0.0
    assert (og[~fin] == 0).all()
    parity.log(f"[decode {tag}] O max abs err {eo:.3e}; LSE max abs err {el:.3e}")
    assert eo <= parity.O_TOL
    assert el <= parity.LSE_TOL


@pytest.mark.parametrize("cfg", CASES, ids=ids)
def test_decode_matches_oracle(cfg):
    B, Hq, Hkv, Nq, Nk, d, m, lk, dt = cfg
    parity.log(f"decode case {ids(cfg)}")
    kw, causal, window = mask_args(m)
    r = si.make_inputs(B, Hq, Hkv, Nk, d, seed=91 + Nk + d, dtype=dt)
    q = si.make_inputs(B, Hq, Hkv, Nq, d, seed=92 + Nq, dtype=dt)["q"]
    inp = {"q": q, "k": r["k"], "v": r["v"]}
    lens = lens_for(lk, B, Nk, Nq, seed=Nk)
    g = parity.to_gpu(inp)
    kv_lens = torch.from_numpy(lens).cuda() if lens is not None else None
    o, lse = ea.decode(g["q"], g["k"], g["v"], kv_lens=kv_lens, **kw)
    torch.cuda.synchronize()
    check(inp, lens, o, lse, ea.default_scale(d), causal, window, ids(cfg))


def test_decode_equals_last_rows_of_forward():
    """Same values, two kernels: decoding the last Nq tokens equals the last
    rows of the causal forward over the whole sequence."""
    B, H, N, d, Nq = 2, 8, 700, 128, 5
    inp = parity.to_gpu(si.make_inputs(B, H, H, N, d, seed=95))
    for kw in (dict(causal=True), dict(window=97), dict(causal=False)):
        o, lse = ea.fwd(inp["q"], inp["k"], inp["v"], **kw)
        od, lsed = ea.decode(inp["q"][:, :, N - Nq:].contiguous(), inp["k"], inp["v"], **kw)
        torch.cuda.synchronize()
        err_o = (od.float() - o[:, :, N - Nq:].float()).abs().max().item()
        err_l = (lsed - lse[:, :, N - Nq:]).abs().max().item()
        parity.log(f"[decode vs fwd {kw}] O {err_o:.3e} LSE {err_l:.3e}")
        assert err_o <= 2 * parity.O_TOL and err_l <= parity.LSE_TOL


def test_decode_cache_views_in_bshd_with_spare_capacity():
    """Caches laid out [B, capacity, Hkv, d] with rows past the filled part
    holding junk; the query and output in BSHD; bit-identical to the
    contiguous call on the filled part."""
    B, Hq, Hkv, Nk, cap, d = 3, 8, 2, 400, 512, 64
    base = si.make_inputs(B, Hq, Hkv, Nk, d, seed=97)
    q = si.make_inputs(B, Hq, Hkv, 1, d, seed=98)["q"].cuda()
    k, v = base["k"].cuda(), base["v"].cuda()
    kc = torch.full((B, cap, Hkv, d), 1e4, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, cap, Hkv, d), -1e4, dtype=torch.bfloat16, device="cuda")
    kc[:, :Nk] = k.transpose(1, 2)
    vc[:, :Nk] = v.transpose(1, 2)
    lens = torch.full((B,), Nk, dtype=torch.int32, device="cuda")
    o1, l1 = ea.decode(q, k, v, causal=True)
    o2, l2 = ea.decode(q.transpose(1, 2).contiguous(), kc, vc, kv_lens=lens, causal=True, layout="bshd")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


def test_decode_errors():
    q = torch.zeros((1, 2, 1, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 10, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        ea.decode(q, k, k, kv_lens=torch.zeros(1, dtype=torch.int64, device="cuda"))
    with pytest.raises(ea.AttnError) as e:
        ea.decode(torch.zeros((1, 3, 1, 64), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((1, 2, 10, 64), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((1, 2, 10, 64), dtype=torch.bfloat16, device="cuda"))
    assert e.value.name == "ATTN_ERR_GQA"


def test_decode_workload_full_shape():
    """The timed decode workload (batch 32, 64 query heads on 8 KV heads,
    4096 cached tokens, d 128), checked on every head of three sequences."""
    w = si.WORKLOADS["c8_decode_70b"]
    inp = si.workload_inputs(w)
    g = parity.to_gpu(inp)
    o, lse = ea.decode(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, window=w.window)
    torch.cuda.synchronize()
    for b in (0, 17, w.B - 1):
        sub = {x: inp[x][b:b + 1] for x in ("q", "k", "v")}
        check(sub, None, o[b:b + 1], lse[b:b + 1], w.scale, w.causal, w.window, f"c8 seq {b}")
