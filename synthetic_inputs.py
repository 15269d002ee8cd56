"""Seeded synthetic workloads shared by the tests, the bench and the oracle runs.

This module only names shapes and draws random numbers; it holds none of the
attention arithmetic. Both the HIP path and the CPU oracle are fed the same
tensors from here.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws Q, K, V
and then dO, in that order (decoding: the K, V cache and then the new Q), as
float32 standard normals, each rounded to bfloat16 (or float16 for fp16
workloads; round to nearest even). Tensors are
returned as contiguous [B, H, N, d]; a BSHD workload hands the same values to
the kernels as contiguous [B, N, H, d].
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    backward: bool
    seed: int
    note: str = field(default="", compare=False)
    window: int | None = None  # sliding window W (keys i-W < j <= i); implies causal
    dtype: str = "bf16"        # "bf16" or "fp16"
    layout: str = "bhsd"       # "bhsd" or "bshd"
    Nq: int | None = None      # decoding: Nq new queries against a cache of N rows
    dropout_p: float = 0.0     # fused dropout probability (seed = workload seed, offset 0)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32, the scale every workload uses."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def pairs(self) -> int:
        """(query, key) pairs per (b, hq): N^2, N(N+1)/2 under the causal mask,
        and sum_i min(i+1, W) under a sliding window of W keys. Decoding: the
        last Nq rows of that count over a full cache of N rows."""
        if self.Nq is not None:
            rows = range(self.N - self.Nq, self.N)
            if self.window is not None:
                return sum(min(i + 1, self.window) for i in rows)
            return sum(i + 1 for i in rows) if self.causal else self.Nq * self.N
        if self.window is not None and self.window < self.N:
            W = self.window
            return W * (W + 1) // 2 + (self.N - W) * W
        return self.N * (self.N + 1) // 2 if self.causal else self.N * self.N

    @property
    def dropout(self):
        """(p, seed, offset) of the dropout stream, or None."""
        if not self.dropout_p:
            return None
        import numpy as np
        return float(np.float32(self.dropout_p)), self.seed, 0

    @property
    def mask(self) -> str:
        if self.window is not None:
            return f"sliding window W={self.window}"
        return "causal" if self.causal else "no mask"

    def fwd_flops(self) -> float:
        """Algorithmic forward flops: two matmuls of 2*d flops per allowed pair."""
        return 4.0 * self.d * self.pairs() * self.B * self.Hq

    def bwd_flops(self) -> float:
        """Algorithmic backward flops: five such matmuls (2.5x the forward)."""
        return 2.5 * self.fwd_flops()

    def fwd_bytes(self) -> float:
        """Read Q, K, V once, write O (16-bit) and LSE (fp32) once."""
        if self.Nq is not None:
            q = self.B * self.Hq * self.Nq * self.d * 2
            kv = 2 * self.B * self.Hkv * self.N * self.d * 2
            return q + kv + q + self.B * self.Hq * self.Nq * 4
        q = self.B * self.Hq * self.N * self.d * 2
        kv = 2 * self.B * self.Hkv * self.N * self.d * 2
        return q + kv + q + self.B * self.Hq * self.N * 4

    def bwd_bytes(self) -> float:
        """Read Q, K, V, O, dO, LSE; write dQ, dK, dV; D row term written once, read twice."""
        q = self.B * self.Hq * self.N * self.d * 2
        kv = self.B * self.Hkv * self.N * self.d * 2
        rows = self.B * self.Hq * self.N * 4
        return 3 * q + 2 * kv + rows + (q + 2 * kv) + 3 * rows


def _w(name, B, Hq, Hkv, N, d, causal, backward, seed, note="", window=None, dtype="bf16",
       layout="bhsd", Nq=None, dropout_p=0.0):
    return Workload(name, B, Hq, Hkv, N, d, causal, backward, seed, note, window, dtype, layout, Nq,
                    dropout_p)


# The five workload families (index k gives seed 1000 + k; the sequence sweep
# adds N). Shapes and distributions as named in the project's headline
# configuration list; the YOLO-like case flattens a 20x20 feature map, as in
# the lpnh.cn YOLO11 article, section 1.2.
WORKLOADS = {
    w.name: w
    for w in [
        _w("c1_yolo_n400", 1, 8, 8, 400, 64, False, False, 1001,
           "YOLO C2PSA-like, 20x20 map flattened"),
        *[
            _w(f"c2_mha_n{n}", 4, 16, 16, n, 64, False, False, 1002 + n,
               "non-causal MHA sequence sweep")
            for n in (512, 1024, 2048, 4096)
        ],
        _w("c3_causal_7b", 2, 32, 32, 4096, 128, True, False, 1003, "7B-like"),
        _w("c4_gqa_70b", 1, 64, 8, 8192, 128, True, False, 1004, "70B-like GQA, G=8"),
        _w("c4_mqa_70b", 1, 64, 1, 8192, 128, True, False, 1004, "MQA, G=64"),
        _w("c4_gqa_70b_bwd", 1, 64, 8, 8192, 128, True, True, 1004,
           "70B-like GQA, G=8, fwd+bwd (dK/dV summed over the group)"),
        _w("c5_bwd_d128", 1, 16, 16, 16384, 128, True, True, 1005, "fwd+bwd"),
        _w("c5_bwd_d80", 1, 16, 16, 4096, 80, True, True, 1005, "fwd+bwd, d=80"),
        # Long-text case for the sliding-window mask (CANN FlashAttention page,
        # mask modes): 16K tokens, a 4096-key band, GQA G=4, fwd+bwd.
        _w("c6_window_d128", 1, 32, 8, 16384, 128, True, True, 1006,
           "fwd+bwd, sliding window 4096, GQA G=4", window=4096),
        # fp16 operands in the [batch, seq, heads, dim] layout (CANN
        # FlashAttention page, tuning section on data types; yunthe.com GQA
        # page, flash_attn_func call): the C5 shape, so the two compare.
        _w("c7_fp16_bshd_d128", 1, 16, 16, 16384, 128, True, True, 1007,
           "fwd+bwd, fp16, BSHD", dtype="fp16", layout="bshd"),
        # One decoding step of the 70B-like GQA model against a full KV cache:
        # batch 32, 4096 cached tokens (the KV-cache example of the yunthe.com
        # GQA page), one new token per sequence.
        _w("c8_decode_70b", 32, 64, 8, 4096, 128, True, False, 1008,
           "decode, 1 new token, KV cache 4096, GQA G=8", Nq=1),
        # Training with the fused dropout of the CANN FlashAttention page's
        # tuning section: the C5 shape with p = 0.1.
        _w("c9_dropout_d128", 1, 16, 16, 16384, 128, True, True, 1009,
           "fwd+bwd, dropout p=0.1", dropout_p=0.1),
    ]
}


TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def make_inputs(B, Hq, Hkv, N, d, seed, with_do=False, dtype="bf16"):
    """Draw Q [B,Hq,N,d], K, V [B,Hkv,N,d] (and dO like Q) on the CPU, in
    bf16 or fp16."""
    t = TORCH_DTYPES[dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32).to(t)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32).to(t)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32).to(t)
    out = {"q": q, "k": k, "v": v}
    if with_do:
        out["do"] = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32).to(t)
    return out


def make_rising_inputs(B, Hq, Hkv, N, d, seed, growth=64.0, v_scale=0.25, with_do=False,
                       dtype="bf16"):
    """Inputs whose key norms grow along the sequence: drawn as make_inputs
    does (float32 normals in the order Q, K, V, dO), then key row j is
    multiplied by 1 + j / growth before the rounding to 16 bits. The spread
    of the scores then widens with the key index, so a row's later key blocks
    reach far larger maxima than its first ones: the recipe that makes a
    running maximum move again and again along a row. V is multiplied by
    v_scale (a power of two, so exactly): with scores this spread a row's
    weights sit on a few keys and O is close to single V rows."""
    t = TORCH_DTYPES[dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    ramp = 1.0 + torch.arange(N, dtype=torch.float32) / float(growth)
    k = k * ramp[None, None, :, None]
    v = v * float(v_scale)
    out = {"q": q.to(t), "k": k.to(t), "v": v.to(t)}
    if with_do:
        out["do"] = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32).to(t)
    return out


def workload_inputs(w: Workload):
    """Q, K, V (and dO) of a workload; for decoding, K and V are the cache
    [B, Hkv, N, d] and Q the Nq new queries, drawn after them."""
    if w.Nq is None:
        return make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, with_do=w.backward, dtype=w.dtype)
    return make_decode_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.N, w.d, w.seed, dtype=w.dtype)


def make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, seed, dtype="bf16"):
    """Draw a K, V cache [B,Hkv,Nk,d] and then Nq new queries Q [B,Hq,Nq,d]."""
    t = TORCH_DTYPES[dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    k = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32).to(t)
    v = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32).to(t)
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32).to(t)
    return {"q": q, "k": k, "v": v}


def in_layout(t: torch.Tensor, layout: str) -> torch.Tensor:
    """A contiguous copy of a [B, H, N, d] tensor in `layout` ("bhsd" returns
    it unchanged, "bshd" gives [B, N, H, d])."""
    return t if layout == "bhsd" else t.transpose(1, 2).contiguous()


def to_f64(t: torch.Tensor):
    """Exact float64 numpy copy of a (bf16 / fp16) CPU or GPU tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


def score_matrix_bytes(B, H, N, elem_bytes):
    """Bytes of one materialised N x N score (or probability) matrix per head,
    over B * H heads: what standard attention writes to memory and the fused
    kernel never does."""
    return B * H * N * N * elem_bytes
