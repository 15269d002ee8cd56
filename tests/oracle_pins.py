"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each check takes the forward / backward implementation as arguments so that the
same checks can be run against deliberately broken copies (see
``test_oracle_mutants.py``) to show that a plausible mistake fails at least one.

Sources of the pinned facts:
* definition of softmax and standard attention: [CANN-FA] (hwcomputing.csdn.net)
  sections on the standard formula/code and on online softmax;
* GQA = MHA on repeat_interleave'd K and V: [FA-GQA] (yunthe.com), GQA class;
* causal mask = current and earlier positions: [CANN-FA] mask modes;
* closed forms and invariants follow from those definitions by algebra.
"""

from __future__ import annotations

import math

import numpy as np

RTOL_EXACT = 1e-12


def rng_arrays(seed, B, Hq, Hkv, N, d, with_do=True, scale_v=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d)) * scale_v
    do = r.standard_normal((B, Hq, N, d)) if with_do else None
    return q, k, v, do


# ---------------------------------------------------------------- brute force

def brute_force_fwd(q, k, v, scale, causal, window=None):
    """Scalar loops straight from the definitions, no max subtraction.

    softmax(x)_j = e^{x_j} / sum_j' e^{x_j'} ([CANN-FA] softmax definition),
    KV head of query head hq = hq // (Hq // Hkv) ([FA-GQA] repeat_interleave).
    Inputs must be small enough that exp() does not overflow.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, Hq, N, d))
    L = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(N):
                weights = []
                for j in range(N):
                    if (causal or window) and j > i:
                        weights.append(0.0)
                        continue
                    if window and j <= i - window:
                        weights.append(0.0)
                        continue
                    s = 0.0
                    for c in range(d):
                        s += float(q[b, h, i, c]) * float(k[b, kv, j, c])
                    weights.append(math.exp(scale * s))
                den = math.fsum(weights)
                L[b, h, i] = math.log(den)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(
                        weights[j] * float(v[b, kv, j, c]) for j in range(N)) / den
    return O, L


def check_brute_force(fwd, seed, B, Hq, Hkv, N, d, causal, scale=0.7):
    q, k, v, _ = rng_arrays(seed, B, Hq, Hkv, N, d, with_do=False)
    O, L = fwd(q, k, v, scale, causal)
    Ob, Lb = brute_force_fwd(q, k, v, scale, causal)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- hand-worked 2 x 2

E = math.e
P_HI = E / (E + 1.0)          # 0.7310585786300049
P_LO = 1.0 / (E + 1.0)        # 0.2689414213699951
DS = 2.0 * E / (E + 1.0) ** 2  # 0.3932238664829637


def hand_2x2_inputs():
    q = np.eye(2)[None, None]
    k = np.eye(2)[None, None]
    v = np.array([[1.0, 2.0], [3.0, 4.0]])[None, None]
    return q, k, v


def check_hand_2x2_fwd(fwd):
    """N=2, d=2, scale=1, Q=K=I, V=[[1,2],[3,4]], worked by hand.

    Scores are the identity, so row 0 weights keys (e, 1)/(e+1) and row 1
    weights (1, e)/(e+1); LSE = ln(e+1). Causal row 0 sees only key 0:
    O_0 = v_0, LSE_0 = s_00 = 1.
    """
    q, k, v = hand_2x2_inputs()
    O, L = fwd(q, k, v, 1.0, False)
    want_o = np.array([[P_HI * 1 + P_LO * 3, P_HI * 2 + P_LO * 4],
                       [P_LO * 1 + P_HI * 3, P_LO * 2 + P_HI * 4]])
    np.testing.assert_allclose(O[0, 0], want_o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(want_o[0], [1.5378828427399902, 2.5378828427399904], atol=1e-15)
    np.testing.assert_allclose(L[0, 0], [math.log(E + 1)] * 2, rtol=0, atol=1e-15)
    Oc, Lc = fwd(q, k, v, 1.0, True)
    np.testing.assert_allclose(Oc[0, 0, 0], [1.0, 2.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Lc[0, 0, 0], 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Oc[0, 0, 1], want_o[1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Lc[0, 0, 1], math.log(E + 1), rtol=0, atol=1e-15)


def check_hand_2x2_bwd(bwd):
    """Same inputs, no mask, dO = [[1,0],[0,0]], worked by hand.

    dV_0 = (P_00, 0), dV_1 = (P_01, 0); dP_0 = (1, 3) so the row term is
    P_00 + 3 P_01 and dS_00 = -dS_01 = -2e/(e+1)^2; dQ_0 = dS_0 K = (dS_00,
    dS_01), dQ_1 = 0; dK_j = dS_0j q_0.
    """
    q, k, v = hand_2x2_inputs()
    do = np.array([[1.0, 0.0], [0.0, 0.0]])[None, None]
    dQ, dK, dV = bwd(q, k, v, do, 1.0, False)
    np.testing.assert_allclose(dV[0, 0], [[P_HI, 0.0], [P_LO, 0.0]], atol=1e-15)
    np.testing.assert_allclose(dQ[0, 0], [[-DS, DS], [0.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(dK[0, 0], [[-DS, 0.0], [DS, 0.0]], atol=1e-15)


# ------------------------------------------------------------- closed forms

def check_zero_queries(fwd, causal):
    """Q = 0: every allowed key gets the same weight, so O_i is the mean of
    the allowed v_j and LSE_i = ln |A_i|."""
    _, k, v, _ = rng_arrays(3, 1, 2, 2, 9, 4, with_do=False)
    q = np.zeros((1, 2, 9, 4))
    O, L = fwd(q, k, v, 0.5, causal)
    for i in range(9):
        n = i + 1 if causal else 9
        np.testing.assert_allclose(O[0, :, i], v[0, :, :n].mean(axis=1), atol=1e-14)
        np.testing.assert_allclose(L[0, :, i], math.log(n), atol=1e-14)


def check_causal_first_row(fwd):
    """Causal row 0 sees only key 0: O_0 = v_0 and LSE_0 = scale <q_0, k_0>."""
    q, k, v, _ = rng_arrays(4, 2, 4, 2, 7, 5, with_do=False)
    O, L = fwd(q, k, v, 0.3, True)
    for b in range(2):
        for h in range(4):
            kv = h // 2
            np.testing.assert_allclose(O[b, h, 0], v[b, kv, 0], atol=1e-14)
            np.testing.assert_allclose(L[b, h, 0], 0.3 * q[b, h, 0] @ k[b, kv, 0], atol=1e-14)


def check_single_key(fwd):
    """N = 1: O = V and LSE = scale <q, k>."""
    q, k, v, _ = rng_arrays(5, 1, 3, 3, 1, 6, with_do=False)
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.9, causal)
        np.testing.assert_allclose(O, v, atol=1e-15)
        np.testing.assert_allclose(L[..., 0], 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                                   atol=1e-14)


def check_identical_keys(fwd):
    """All keys equal: weights are uniform whatever the queries are."""
    q, k, v, _ = rng_arrays(6, 1, 2, 1, 8, 3, with_do=False)
    k[:] = k[:, :, :1]
    O, _ = fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (8, 3)), atol=1e-14)


def check_gqa_is_repeated_mha(fwd, bwd, G, Hkv=2, causal=True):
    """[FA-GQA]: GQA equals MHA on K, V repeat_interleave'd n_rep = G times
    along the head axis; the K/V gradients of GQA are the sums of the MHA
    gradients over each group of G heads."""
    Hq = G * Hkv
    q, k, v, do = rng_arrays(7 + G, 2, Hq, Hkv, 11, 4)
    O, L = fwd(q, k, v, 0.6, causal)
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    Om, Lm = fwd(q, kr, vr, 0.6, causal)
    np.testing.assert_allclose(O, Om, atol=1e-14)
    np.testing.assert_allclose(L, Lm, atol=1e-14)
    dQ, dK, dV = bwd(q, k, v, do, 0.6, causal)
    dQm, dKm, dVm = bwd(q, kr, vr, do, 0.6, causal)
    np.testing.assert_allclose(dQ, dQm, atol=1e-13)
    np.testing.assert_allclose(dK, dKm.reshape(2, Hkv, G, 11, 4).sum(2), atol=1e-13)
    np.testing.assert_allclose(dV, dVm.reshape(2, Hkv, G, 11, 4).sum(2), atol=1e-13)


def check_library_softmax(fwd, causal):
    """Special case of a library routine: torch float64 on the CPU of the
    standard attention code ([CANN-FA]), softmax(Q K^T * scale + mask) V."""
    import torch
    q, k, v, _ = rng_arrays(8, 2, 4, 4, 33, 16, with_do=False)
    O, L = fwd(q, k, v, 0.25, causal)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-2, -1).contiguous()) * 0.25
    if causal:
        s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    np.testing.assert_allclose(O, o.numpy(), atol=1e-13)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-13)


# --------------------------------------------------------------- invariants

def check_key_shift(fwd, causal):
    """Adding c to every k_j leaves O unchanged and shifts LSE_i by
    scale <q_i, c> (every score of row i moves by the same amount)."""
    q, k, v, _ = rng_arrays(9, 1, 2, 2, 13, 5, with_do=False)
    c = np.random.default_rng(10).standard_normal(5)
    O, L = fwd(q, k, v, 0.4, causal)
    O2, L2 = fwd(q, k + c, v, 0.4, causal)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2 - L, 0.4 * q @ c, atol=1e-13)


def check_value_shift(fwd, causal):
    """Adding c to every v_j adds c to every O_i (weights sum to 1)."""
    q, k, v, _ = rng_arrays(11, 1, 2, 2, 13, 5, with_do=False)
    c = np.arange(5.0) - 2
    O, _ = fwd(q, k, v, 0.4, causal)
    O2, _ = fwd(q, k, v + c, 0.4, causal)
    np.testing.assert_allclose(O2, O + c, atol=1e-13)


def check_convex_hull(fwd, causal):
    """Each O_ic lies between min and max of v_jc over the allowed keys."""
    q, k, v, _ = rng_arrays(12, 1, 2, 1, 17, 4, with_do=False)
    O, _ = fwd(q, k, v, 2.0, causal)
    for i in range(17):
        n = i + 1 if causal else 17
        lo = v[0, 0, :n].min(0)
        hi = v[0, 0, :n].max(0)
        assert np.all(O[0, :, i] >= lo - 1e-14) and np.all(O[0, :, i] <= hi + 1e-14)


def check_key_permutation(fwd):
    """No mask: permuting keys together with values changes nothing."""
    q, k, v, _ = rng_arrays(13, 1, 2, 2, 15, 4, with_do=False)
    perm = np.random.default_rng(14).permutation(15)
    O, L = fwd(q, k, v, 0.5, False)
    O2, L2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)


def check_rows_sum_to_one(fwd_head, causal):
    """Every row of the materialised P sums to 1 and is 0 off the mask."""
    q, k, v, _ = rng_arrays(15, 1, 1, 1, 20, 6, with_do=False)
    _, _, S, P = fwd_head(q[0, 0], k[0, 0], v[0, 0], 0.8, causal, 0, True)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)
    if causal:
        assert np.all(P[np.triu_indices(20, 1)] == 0.0)


def check_bwd_identities(bwd, causal):
    """Gradient identities of the definition:
    * sum_j dK_j = 0 per (b, hkv): shifting every key by c leaves O unchanged;
    * sum_j dV_j = sum over the group's query heads and rows of dO_i
      (rows of P sum to 1);
    * the gradients are linear in dO."""
    q, k, v, do = rng_arrays(16, 2, 4, 2, 12, 5)
    dQ, dK, dV = bwd(q, k, v, do, 0.7, causal)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(axis=2), do.reshape(2, 2, 2, 12, 5).sum(axis=(2, 3)),
                               atol=1e-12)
    do2 = np.random.default_rng(17).standard_normal(do.shape)
    g1 = bwd(q, k, v, do2, 0.7, causal)
    g12 = bwd(q, k, v, 2.0 * do - 3.0 * do2, 0.7, causal)
    for a, b_, c in zip((dQ, dK, dV), g1, g12):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b_, atol=1e-12)


def check_finite_differences(fwd, bwd, causal, seed=18, B=1, Hq=2, Hkv=1, N=5, d=3):
    """Central differences of L = sum(O * dO) for every element of Q, K, V."""
    scale = 0.9
    q, k, v, do = rng_arrays(seed, B, Hq, Hkv, N, d)
    dQ, dK, dV = bwd(q, k, v, do, scale, causal)
    h = 1e-6

    def loss(qq, kk, vv):
        O, _ = fwd(qq, kk, vv, scale, causal)
        return float(np.sum(O * do))

    for arr, grad, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert err < 1e-7, f"finite-difference mismatch on input {which}: rel err {err:.3e}"


def check_blockwise_equals_plain(blockwise, fwd_head, causal, N=70, d=8):
    """The blockwise online-softmax loop equals the materialising definition
    for any block sizes ([YOLO11-FA2] section 2.2, [CANN-FA] online softmax:
    the result is exact up to summation order)."""
    q, k, v, _ = rng_arrays(19, 1, 1, 1, N, d, with_do=False)
    q, k, v = q[0, 0] * 2.0, k[0, 0], v[0, 0]
    O, L = fwd_head(q, k, v, 0.5, causal)
    for br, bc in ((1, 1), (7, 7), (64, 64), (N, N), (16, 5)):
        Ob, Lb = blockwise(q, k, v, 0.5, causal, br, bc)
        np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-12)


def all_forward_checks(fwd):
    """Every forward pin that needs only the [B,H,N,d] forward entry point."""
    check_brute_force(fwd, 1, 1, 2, 1, 5, 3, False)
    check_brute_force(fwd, 2, 2, 4, 2, 6, 4, True)
    check_hand_2x2_fwd(fwd)
    for causal in (False, True):
        check_zero_queries(fwd, causal)
        check_key_shift(fwd, causal)
        check_value_shift(fwd, causal)
        check_convex_hull(fwd, causal)
        check_library_softmax(fwd, causal)
    check_causal_first_row(fwd)
    check_single_key(fwd)
    check_identical_keys(fwd)
    check_key_permutation(fwd)


def all_backward_checks(fwd, bwd):
    check_hand_2x2_bwd(bwd)
    for causal in (False, True):
        check_bwd_identities(bwd, causal)
        check_finite_differences(fwd, bwd, causal)
    for G in (1, 2, 3):
        check_gqa_is_repeated_mha(fwd, bwd, G)


# --------------------------------------------------------- sliding window

def check_window_brute_force(fwd_w, seed, B, Hq, Hkv, N, d, window, scale=0.7):
    """[CANN-FA] sliding-window mask mode: keys i - W < j <= i only."""
    q, k, v, _ = rng_arrays(seed, B, Hq, Hkv, N, d, with_do=False)
    O, L = fwd_w(q, k, v, scale, window)
    Ob, Lb = brute_force_fwd(q, k, v, scale, True, window)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-13)


def check_window_special_cases(fwd, fwd_w):
    """W = 1: each row sees only itself (O_i = v_i, LSE_i = s_ii). W >= N: the
    plain causal mask. Q = 0: O_i is the mean of the last min(i+1, W) values
    and LSE_i = ln min(i+1, W)."""
    q, k, v, _ = rng_arrays(20, 1, 2, 1, 12, 5, with_do=False)
    O, L = fwd_w(q, k, v, 0.6, 1)
    np.testing.assert_allclose(O, np.repeat(v, 2, axis=1), atol=1e-14)
    np.testing.assert_allclose(L, 0.6 * np.einsum("bhnd,bhnd->bhn", q, np.repeat(k, 2, axis=1)), atol=1e-13)
    for W in (12, 13, 100):
        Ow, Lw = fwd_w(q, k, v, 0.6, W)
        Oc, Lc = fwd(q, k, v, 0.6, True)
        np.testing.assert_allclose(Ow, Oc, atol=1e-15)
        np.testing.assert_allclose(Lw, Lc, atol=1e-15)
    z = np.zeros_like(q)
    O, L = fwd_w(z, k, v, 0.6, 4)
    for i in range(12):
        lo = max(0, i - 3)
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, lo:i + 1].mean(0), atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], np.log(i + 1 - lo), atol=1e-14)


def check_window_blockwise(blockwise, fwd_head):
    q, k, v, _ = rng_arrays(21, 1, 1, 1, 70, 8, with_do=False)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    for W in (1, 5, 33):
        O, L = fwd_head(q, k, v, 0.5, True, window=W)
        for br, bc in ((1, 1), (7, 7), (16, 5), (64, 64)):
            Ob, Lb = blockwise(q, k, v, 0.5, True, br, bc, window=W)
            np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-12)
            np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-12)


def check_window_gradients(fwd_w, bwd_w):
    """Finite differences and the key-shift / value-sum identities under the
    window mask (every row still has at least one key: itself)."""
    scale, W = 0.9, 3
    q, k, v, do = rng_arrays(22, 1, 2, 1, 6, 3)
    dQ, dK, dV = bwd_w(q, k, v, do, scale, W)
    h = 1e-6

    def loss(qq, kk, vv):
        O, _ = fwd_w(qq, kk, vv, scale, W)
        return float(np.sum(O * do))

    for arr, grad, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a_p = [q.copy(), k.copy(), v.copy()]
            a_m = [q.copy(), k.copy(), v.copy()]
            a_p[which][idx] += h
            a_m[which][idx] -= h
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        assert np.linalg.norm(num - grad) / np.linalg.norm(grad) < 1e-7
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(axis=2), do.sum(axis=(1, 2))[:, None], atol=1e-12)


# ------------------------------------------------------------------- decoding

def brute_force_decode(q, k, v, scale, causal, kv_lens, window=None):
    """Scalar loops: query i of sequence b at position L_b - Nq + i, keys
    j < L_b, the causal / window tests written out per pair, e^x / sum e^x
    with no max subtraction; a query with no key gets O = 0, LSE = -inf."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Nq, d))
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        Lb = min(max(int(kv_lens[b]), 0), Nk)
        for h in range(Hq):
            kv = h // G
            for i in range(Nq):
                pos = Lb - Nq + i
                w = []
                for j in range(Lb):
                    ok = True
                    if (causal or window) and j > pos:
                        ok = False
                    if window and j <= pos - window:
                        ok = False
                    if ok:
                        s = sum(float(q[b, h, i, c]) * float(k[b, kv, j, c]) for c in range(d))
                        w.append((j, math.exp(scale * s)))
                if not w:
                    continue
                den = math.fsum(x for _, x in w)
                L[b, h, i] = math.log(den)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(x * float(v[b, kv, j, c]) for j, x in w) / den
    return O, L


def check_decode_brute_force(dec, seed, causal, window=None):
    r = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 3, 9, 5
    q = r.standard_normal((B, Hq, Nq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    lens = [9, 5, 2]  # full cache, partly filled, shorter than Nq
    O, L = dec(q, k, v, 0.6, causal, lens, window)
    Ob, Lb = brute_force_decode(q, k, v, 0.6, causal, lens, window)
    np.testing.assert_allclose(O, Ob, rtol=RTOL_EXACT, atol=1e-13)
    np.testing.assert_array_equal(np.isfinite(L), np.isfinite(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=RTOL_EXACT, atol=1e-13)


def check_decode_is_last_rows(dec, fwd_full, causal, window=None):
    """Decoding the last Nq tokens of a sequence gives the last Nq rows of
    self-attention over it (the alignment rule), for every mask kind."""
    r = np.random.default_rng(31)
    B, Hq, Hkv, N, d, Nq = 2, 4, 2, 11, 6, 4
    Q = r.standard_normal((B, Hq, N, d))
    K = r.standard_normal((B, Hkv, N, d))
    V = r.standard_normal((B, Hkv, N, d))
    O, L = fwd_full(Q, K, V, 0.8, causal, window)
    Od, Ld = dec(Q[:, :, N - Nq:], K, V, 0.8, causal, None, window)
    np.testing.assert_allclose(Od, O[:, :, N - Nq:], rtol=RTOL_EXACT, atol=1e-13)
    np.testing.assert_allclose(Ld, L[:, :, N - Nq:], rtol=RTOL_EXACT, atol=1e-13)
    # per-sequence lengths: a cache padded with junk beyond L_b changes nothing
    pad = r.standard_normal((B, Hkv, 5, d)) * 1e3
    Kp = np.concatenate([K, pad], axis=2)
    Vp = np.concatenate([V, pad], axis=2)
    Od2, Ld2 = dec(Q[:, :, N - Nq:], Kp, Vp, 0.8, causal, [N, N], window)
    np.testing.assert_allclose(Od2, Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ld2, Ld, rtol=0, atol=1e-13)


def check_decode_special_cases(dec):
    """One new token sees the whole cache under either mask; an empty cache or
    a query before the first cached position sees nothing."""
    r = np.random.default_rng(33)
    q = r.standard_normal((2, 2, 1, 4))
    k = r.standard_normal((2, 1, 6, 4))
    v = r.standard_normal((2, 1, 6, 4))
    a = dec(q, k, v, 0.5, False, [6, 3], None)
    c = dec(q, k, v, 0.5, True, [6, 3], None)
    np.testing.assert_allclose(a[0], c[0], atol=1e-15)
    np.testing.assert_allclose(a[1], c[1], atol=1e-15)
    # Q = 0: O is the mean of the visible values, LSE = ln(count)
    z = np.zeros_like(q)
    O, L = dec(z, k, v, 0.5, True, [6, 3], 4)
    np.testing.assert_allclose(O[0, :, 0], np.repeat(v[0, :, 2:6].mean(axis=1), 2, axis=0), atol=1e-14)
    np.testing.assert_allclose(L[0], np.log(4), atol=1e-14)
    np.testing.assert_allclose(O[1, :, 0], np.repeat(v[1, :, 0:3].mean(axis=1), 2, axis=0), atol=1e-14)
    np.testing.assert_allclose(L[1], np.log(3), atol=1e-14)
    O, L = dec(q, k, v, 0.5, True, [0, 7], None)  # empty cache; length clamped to Nk
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    O6, L6 = dec(q, k, v, 0.5, True, [6, 6], None)
    np.testing.assert_allclose(O[1], O6[1], atol=0)
    q3 = r.standard_normal((1, 1, 3, 4))
    O8, L8 = dec(q3, k[:1], v[:1], 0.5, True, [8], None)  # 8 > Nk = 6 is clamped to 6
    O6, L6 = dec(q3, k[:1], v[:1], 0.5, True, [6], None)
    np.testing.assert_allclose(O8, O6, atol=0)
    np.testing.assert_allclose(L8, L6, atol=0)
    O, L = dec(q3, k[:1], v[:1], 0.5, True, [2], None)  # L_b = 2 < Nq = 3
    assert np.all(O[0, 0, 0] == 0) and np.isneginf(L[0, 0, 0])
    assert np.all(np.isfinite(L[0, 0, 1:]))


# ------------------------------------------------------------ Philox, dropout

def check_philox_against_numpy(philox):
    """The generic Philox-4xW-R at W = 64, R = 10 equals numpy's Philox bit
    generator (a library implementation of the same published function);
    numpy advances its 256-bit counter by one before producing each block."""
    r = np.random.default_rng(7)
    for _ in range(5):
        key = [int(x) for x in r.integers(0, 2**63, size=2, dtype=np.uint64)]
        ctr = [int(x) for x in r.integers(0, 2**63, size=4, dtype=np.uint64)]
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
        got = bg.random_raw(8)
        for blk in range(2):
            c = list(ctr)
            c[0] += blk + 1  # no carry: ctr[0] < 2^63
            want = philox(c, key, rounds=10, width=64)
            assert [int(x) for x in want] == [int(x) for x in got[4 * blk:4 * blk + 4]]


def check_philox_weyl_constants(constants):
    """The Weyl constants by which Philox advances its key are the golden
    ratio and sqrt(3), less one, as binary fractions of the word size
    (Salmon et al., SC'11, section 3.3): W0 = floor(2^W (phi - 1)) and
    W1 = floor(2^W (sqrt(3) - 1)). Integer square roots make both exact; the
    32-bit constants are the top halves of the 64-bit ones (which the numpy
    pin covers)."""
    for w in (32, 64):
        one = 1 << w
        phi_m1 = (math.isqrt(5 << (2 * w)) - one) // 2   # floor(2^w (sqrt(5) - 1) / 2)
        sqrt3_m1 = math.isqrt(3 << (2 * w)) - one         # floor(2^w (sqrt(3) - 1))
        assert constants[w]["W0"] == phi_m1, w
        assert constants[w]["W1"] == sqrt3_m1, w
    assert constants[32]["W0"] == constants[64]["W0"] >> 32
    assert constants[32]["W1"] == constants[64]["W1"] >> 32


def check_philox32_against_rocrand(philox4x32, run_rocrand):
    """Philox-4x32-10 equals rocRAND's philox4x32_10_engine (an independent
    library implementation) on random 128-bit counters and 64-bit keys:
    this pins the two 32-bit multipliers, which have no closed form.
    `run_rocrand` maps lines "seed counter_lo64 counter_hi64" to the four
    words of each block."""
    r = np.random.default_rng(9)
    cases = [(0, 0, 0), (2**64 - 1, 2**62 - 1, 2**64 - 1)]
    for _ in range(40):
        seed = int(r.integers(0, 2**63, dtype=np.uint64)) * 2 + int(r.integers(0, 2))
        lo = int(r.integers(0, 2**62, dtype=np.uint64))
        hi = int(r.integers(0, 2**63, dtype=np.uint64)) * 2 + int(r.integers(0, 2))
        cases.append((seed, lo, hi))
    got = run_rocrand(cases)
    for (seed, lo, hi), words in zip(cases, got):
        m = 0xFFFFFFFF
        want = philox4x32((lo & m, lo >> 32, hi & m, hi >> 32), (seed & m, seed >> 32), rounds=10)
        assert [int(x) for x in want] == words, (seed, lo, hi)


def check_philox32_stream(philox, philox4x32):
    """The vectorised 32-bit path equals the generic one, and its words look
    uniform: mean, per-bit frequencies and lag-1 correlation within 5 sigma."""
    r = np.random.default_rng(8)
    c = [r.integers(0, 2**32, size=2000, dtype=np.uint64) for _ in range(4)]
    a = philox(c, (11, 22), rounds=10, width=32)
    b = philox4x32(c, (11, 22), rounds=10)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    n = 1 << 18
    j = np.arange(n)
    w = np.concatenate(philox4x32((j, 0, 5, 9), (123, 456))).astype(np.float64)
    u = w / 2.0**32
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
    bits = ((w.astype(np.uint64)[:, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(w.size))
    cc = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(cc) < 5 / np.sqrt(u.size)
    # rounds = 0 is the identity on the counter
    z = philox4x32((1, 2, 3, 4), (5, 6), rounds=0)
    assert [int(x) for x in z] == [1, 2, 3, 4]


def _p_realised(p):
    """Drop probability of a 16-bit threshold floor(p * 2^16)."""
    return math.floor(float(p) * 65536.0) / 65536.0


def check_keep_mask(dropout_keep, keep_threshold):
    """Keep fraction 1 - p (5 sigma), p = 0 keeps everything, masks depend on
    head, seed and offset, and are reproducible; the two keys that share a
    Philox word (its two 16-bit halves) decide independently."""
    assert keep_threshold(0.0) == 0 and keep_threshold(0.5) == 2**15
    assert keep_threshold(np.float32(0.1)) == int(np.floor(np.float64(np.float32(0.1)) * 2**16))
    assert keep_threshold(1.0 - 2.0**-20) == 65535
    both = dropout_keep(5, np.arange(256), np.arange(512), 0.5, 99, 1)
    pair = both[:, 0::2] & both[:, 1::2]
    sd = np.sqrt(0.25 * 0.75 / pair.size)
    assert abs(pair.mean() - 0.25) < 5 * sd
    # rows of one query quad (different words of one block) agree half the time
    agree = both[0::4] == both[1::4]
    sd = np.sqrt(0.25 / agree.size)
    assert abs(agree.mean() - 0.5) < 5 * sd
    for p in (0.1, 0.5, 0.9):
        m = dropout_keep(3, np.arange(512), np.arange(512), p, 1234, 7)
        sd = np.sqrt(p * (1 - p) / m.size)
        assert abs(m.mean() - (1 - p)) < 5 * sd
    assert dropout_keep(0, np.arange(8), np.arange(8), 0.0, 1, 2).all()
    a = dropout_keep(3, np.arange(64), np.arange(64), 0.5, 1234, 7)
    assert np.array_equal(a, dropout_keep(3, np.arange(64), np.arange(64), 0.5, 1234, 7))
    for other in (dropout_keep(4, np.arange(64), np.arange(64), 0.5, 1234, 7),
                  dropout_keep(3, np.arange(64), np.arange(64), 0.5, 1235, 7),
                  dropout_keep(3, np.arange(64), np.arange(64), 0.5, 1234, 8),
                  dropout_keep(3, np.arange(64), np.arange(64), 0.5, 1234 + (1 << 32), 7)):
        assert 0.3 < (a != other).mean() < 0.7
    # rows and columns are addressed absolutely (sub-blocks agree)
    sub = dropout_keep(3, np.arange(10, 30), np.arange(5, 40), 0.5, 1234, 7)
    assert np.array_equal(sub, a[10:30, 5:40])


def brute_force_dropout_fwd(q, k, v, scale, causal, keep_of, p):
    """Scalar loops: O_i = sum_j e^{s_ij} m_ij v_j / ((1 - p) sum_j e^{s_ij}),
    LSE_i = ln sum_j e^{s_ij} (dropout does not touch the normaliser)."""
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    O = np.zeros((B, Hq, N, d))
    L = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            m = keep_of(b * Hq + h, N)
            for i in range(N):
                e = [math.exp(scale * sum(float(q[b, h, i, c]) * float(k[b, kv, j, c]) for c in range(d)))
                     if not (causal and j > i) else 0.0 for j in range(N)]
                den = math.fsum(e)
                L[b, h, i] = math.log(den)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(e[j] * (1.0 if m[i, j] else 0.0) * float(v[b, kv, j, c])
                                              for j in range(N)) / ((1.0 - p) * den)
    return O, L


def check_dropout_forward(fwd_d, fwd, dropout_keep):
    p, seed, off = 0.3, 99, 5
    q, k, v, _ = rng_arrays(60, 2, 4, 2, 7, 3, with_do=False)
    for causal in (False, True):
        O, L = fwd_d(q, k, v, 0.7, causal, (p, seed, off))
        Ob, Lb = brute_force_dropout_fwd(q, k, v, 0.7, causal,
                                         lambda bh, N: dropout_keep(bh, np.arange(N), np.arange(N), p, seed, off),
                                         _p_realised(p))
        np.testing.assert_allclose(O, Ob, rtol=RTOL_EXACT, atol=1e-13)
        np.testing.assert_allclose(L, Lb, rtol=RTOL_EXACT, atol=1e-13)
        O0, L0 = fwd_d(q, k, v, 0.7, causal, (0.0, seed, off))
        Oc, Lc = fwd(q, k, v, 0.7, causal)
        np.testing.assert_allclose(O0, Oc, atol=1e-15)
        np.testing.assert_allclose(L0, Lc, atol=1e-15)


def check_dropout_expectation(fwd_d, fwd):
    """E[M / (1 - p)] = 1: the mean of O over many seeds tends to the
    no-dropout output (checked to 6 standard errors)."""
    q, k, v, _ = rng_arrays(61, 1, 1, 1, 5, 2, with_do=False)
    Oc, _ = fwd(q, k, v, 0.5, True)
    outs = np.stack([fwd_d(q, k, v, 0.5, True, (0.4, s, 0))[0] for s in range(1500)])
    se = outs.std(axis=0) / np.sqrt(outs.shape[0]) + 1e-12
    assert np.all(np.abs(outs.mean(axis=0) - Oc) < 6 * se)


def check_dropout_gradients(fwd_d, bwd_d):
    """Finite differences of sum(O * dO) for a fixed mask (seed, offset) give
    the backward under dropout, GQA with two heads per KV head."""
    scale, drop = 0.8, (0.35, 4242, 3)
    q, k, v, do = rng_arrays(62, 1, 2, 1, 6, 3)
    for causal in (False, True):
        dQ, dK, dV = bwd_d(q, k, v, do, scale, causal, drop)
        h = 1e-6

        def loss(qq, kk, vv):
            O, _ = fwd_d(qq, kk, vv, scale, causal, drop)
            return float(np.sum(O * do))

        for arr, grad, which in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
            num = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                a_p = [q.copy(), k.copy(), v.copy()]
                a_m = [q.copy(), k.copy(), v.copy()]
                a_p[which][idx] += h
                a_m[which][idx] -= h
                num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
            assert np.linalg.norm(num - grad) / np.linalg.norm(grad) < 1e-7
        np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
