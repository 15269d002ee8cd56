"""Helpers for GPU-vs-oracle parity (imported by the gpu tests only).

Tolerances (stated for bf16 inputs with fp32 accumulation):
  O:      max |O_gpu - O_ref|                      <= 1e-2
  LSE:    max |LSE_gpu - LSE_ref|                  <= 1e-3
  dQ, dK, dV: ||g_gpu - g_ref||_2 / ||g_ref||_2    <= 2e-2  (each tensor)
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
import synthetic_inputs as si

O_TOL = 1e-2
LSE_TOL = 1e-3
GRAD_TOL = 2e-2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_gpu(inputs):
    return {k: v.cuda() for k, v in inputs.items()}


def rel_l2(g, r):
    den = max(float(np.linalg.norm(r)), 1e-3 * np.sqrt(r.size))
    return float(np.linalg.norm(g - r)) / den


def check_fwd(inputs_cpu, o_gpu, lse_gpu, scale, causal, heads, tag="", window=None, dropout=None):
    q, k, v = (si.to_f64(inputs_cpu[x]) for x in ("q", "k", "v"))
    O, L = oracle.ref_fwd(q, k, v, scale, causal, heads=heads, window=window, dropout=dropout)
    # Under dropout kept weights are scaled by 1/(1-p), so |O| can leave the
    # range of V; the 16-bit output rounding (2^-8 |O| for bf16) is added.
    rel = 0.0 if dropout is None else 2.0 ** -8
    og = si.to_f64(o_gpu)
    lg = lse_gpu.detach().cpu().double().numpy()
    worst_o, worst_l = 0.0, 0.0
    for b, h in heads:
        eo = np.abs(og[b, h] - O[b, h]) - rel * np.abs(O[b, h])
        el = np.abs(lg[b, h] - L[b, h])
        if eo.max() >= worst_o:
            worst_o = float(eo.max())
            where_o = (b, h) + np.unravel_index(eo.argmax(), eo.shape)
        if el.max() >= worst_l:
            worst_l = float(el.max())
            where_l = (b, h, int(el.argmax()))
    log(f"[fwd {tag}] O max abs err {worst_o:.3e} at {where_o}; LSE max abs err {worst_l:.3e} at {where_l}")
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert worst_o <= O_TOL, f"O error {worst_o} at {where_o}"
    assert worst_l <= LSE_TOL, f"LSE error {worst_l} at {where_l}"
    return worst_o, worst_l


def check_bwd(inputs_cpu, grads_gpu, scale, causal, kv_heads, Hq, Hkv, tag="", window=None,
              dropout=None):
    q, k, v, do = (si.to_f64(inputs_cpu[x]) for x in ("q", "k", "v", "do"))
    dQ, dK, dV = oracle.ref_bwd(q, k, v, do, scale, causal, kv_heads=kv_heads, window=window,
                                dropout=dropout)
    G = Hq // Hkv
    gq, gk, gv = (si.to_f64(t) for t in grads_gpu)
    errs = {}
    for name, g, r in (("dQ", gq, dQ), ("dK", gk, dK), ("dV", gv, dV)):
        sel_g, sel_r = [], []
        for b, hk in kv_heads:
            if name == "dQ":
                sel_g.append(g[b, hk * G:(hk + 1) * G])
                sel_r.append(r[b, hk * G:(hk + 1) * G])
            else:
                sel_g.append(g[b, hk])
                sel_r.append(r[b, hk])
        gg, rr = np.stack(sel_g), np.stack(sel_r)
        assert np.isfinite(gg).all(), f"{name} has non-finite values"
        errs[name] = rel_l2(gg, rr)
    log(f"[bwd {tag}] rel L2: " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= GRAD_TOL, f"{name} rel L2 error {e}"
    return errs
