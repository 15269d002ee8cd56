"""Plain fp64 reference of exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Everything here materialises the score matrix S and the probability matrix P
(row-chunked so that one head of length 16384 fits in host memory: every row
is still computed over all of its keys at once) and works in float64 on the
exact values of the inputs. Arrays use the contiguous [batch, heads, seq, dim]
layout that the [CANN-FA] usage example and the [YOLO11-FA2] section 3.2 code
comment both give for Q, K, V.

Notation: per (b, hq), query rows i and key rows j in [0, N); G = Hq / Hkv;
hkv = hq // G; s_ij = scale * <q_i, k_j>; the allowed key set A_i is all j < N
(no mask), j <= i (causal mask) or i - W < j <= i (sliding window of W keys).
"""

from __future__ import annotations

import numpy as np

from .philox import dropout_keep, effective_p

__all__ = [
    "kv_head_of",
    "allowed_mask",
    "ref_fwd_head",
    "ref_fwd",
    "ref_bwd_group",
    "ref_bwd",
    "blockwise_online_fwd",
    "ref_decode",
]

DEFAULT_CHUNK = 1024


def kv_head_of(hq: int, Hq: int, Hkv: int) -> int:
    """KV head used by query head ``hq``.

    [FA-GQA], GQA class: K and V are expanded with
    ``repeat_interleave(n_rep, dim=1)``, n_rep = Hq // Hkv, so expanded head
    hq holds original KV head hq // n_rep (consecutive grouping). MQA is
    Hkv = 1, MHA is Hkv = Hq (same page, GQA section).
    """
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return hq // (Hq // Hkv)


def allowed_mask(row0: int, nrows: int, N: int, causal: bool, window=None) -> np.ndarray:
    """Boolean [nrows, N]: True where key j may be attended by query row0+r.

    [CANN-FA], tuning section on mask modes: the causal mask looks only at
    positions before the current one (the current one included, since a
    query always sees itself in self-attention); the sliding-window mask
    looks only at the most recent `window` positions, i.e. keys
    i - window + 1 <= j <= i (it implies the causal mask); no mask looks at
    everything.
    """
    if window is not None and window < 1:
        raise ValueError("window must be >= 1")
    if not causal and window is None:
        return np.ones((nrows, N), dtype=bool)
    i = np.arange(row0, row0 + nrows)[:, None]
    j = np.arange(N)[None, :]
    ok = j <= i
    if window is not None:
        ok &= j > i - window
    return ok


def _scores(q, k, scale, row0, causal, window=None):
    # [CANN-FA] standard attention code, step 1: scores = Q @ K^T / sqrt(d_k);
    # the scale is an explicit argument so that any value can be checked.
    S = (q @ k.T) * scale
    mask = allowed_mask(row0, q.shape[0], k.shape[0], causal, window)
    return np.where(mask, S, -np.inf)


def _softmax_rows(S):
    """Row softmax and row log-sum-exp of a masked score block.

    [CANN-FA] softmax definition: softmax(x_i) = e^{x_i} / sum_j e^{x_j}.
    Subtracting the row maximum first changes nothing mathematically and
    keeps exp() finite. LSE_i = ln sum_j exp(s_ij) over the allowed keys.
    A row with no allowed key (cannot happen for self-attention) gets P = 0
    and LSE = -inf.
    """
    m = S.max(axis=1)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - safe_m[:, None])
    den = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(den[:, None] > 0, E / den[:, None], 0.0)
        lse = np.where(den > 0, safe_m + np.log(den), -np.inf)
    return P, lse


def _dropped(P, keep, p_drop):
    """Attention weights after dropout: kept entries scaled by 1 / (1 - p),
    dropped ones zero ([CANN-FA] tuning section: dropout applied inside the
    fused kernel, on the attention weights, during training)."""
    if keep is None:
        return P
    return np.where(keep, P / (1.0 - p_drop), 0.0)


def _keep_rows(dropout, bh, r0, r1, N):
    """Keep mask of rows r0..r1-1 of head bh under dropout = (p, seed, offset),
    and the drop probability the mask realises (p rounded down to a multiple
    of 2^-16), by which the kept weights are rescaled."""
    if dropout is None:
        return None, 0.0
    p, seed, offset = dropout
    return dropout_keep(bh, np.arange(r0, r1), np.arange(N), p, seed, offset), effective_p(p)


def ref_fwd_head(q, k, v, scale, causal=False, row0=0, return_sp=False, window=None, keep=None,
                 p_drop=0.0):
    """Forward of one head for query rows row0 .. row0+len(q)-1.

    q: [R, d]; k, v: [N, d]. Returns O [R, d] and LSE [R] (float64), plus S and
    P [R, N] when ``return_sp``. [CANN-FA] standard attention code:
    scores -> softmax -> attn_weights @ V, with S and P materialised. With a
    boolean ``keep`` mask [R, N], the weights go through dropout of
    probability ``p_drop`` before the product with V; LSE and the returned P
    are those of the softmax itself.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S = _scores(q, k, scale, row0, causal, window)
    P, lse = _softmax_rows(S)
    O = _dropped(P, keep, p_drop) @ v
    if return_sp:
        return O, lse, S, P
    return O, lse


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, Hq, Hkv, N, d


def ref_fwd(q, k, v, scale, causal=False, heads=None, chunk=DEFAULT_CHUNK, window=None,
            dropout=None):
    """Forward for [B, Hq, N, d] query and [B, Hkv, N, d] key/value arrays.

    Returns (O [B, Hq, N, d], LSE [B, Hq, N]) in float64. ``heads`` restricts
    the work to a list of (b, hq) pairs; other entries are left NaN. Rows are
    processed ``chunk`` at a time; each chunk still holds full rows of S, P
    ([YOLO11-FA2] section 3.2 loops over blocks of query rows the same way and
    applies a full-row softmax to each block). ``dropout`` = (p, seed, offset)
    applies dropout with the keep mask of ``philox.dropout_keep`` for head
    bh = b * Hq + hq.
    """
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    O = np.full((B, Hq, N, d), np.nan)
    LSE = np.full((B, Hq, N), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in heads:
        hkv = kv_head_of(hq, Hq, Hkv)
        kk = np.asarray(k[b, hkv], dtype=np.float64)
        vv = np.asarray(v[b, hkv], dtype=np.float64)
        for r0 in range(0, N, chunk):
            r1 = min(N, r0 + chunk)
            keep, p = _keep_rows(dropout, b * Hq + hq, r0, r1, N)
            o, lse = ref_fwd_head(q[b, hq, r0:r1], kk, vv, scale, causal, row0=r0, window=window,
                                  keep=keep, p_drop=p)
            O[b, hq, r0:r1] = o
            LSE[b, hq, r0:r1] = lse
    return O, LSE


def ref_bwd_group(q, k, v, do, scale, causal=False, chunk=DEFAULT_CHUNK, window=None, dropout=None):
    """Backward of one KV head and the G query heads that share it.

    q, do: [G, N, d] (the query heads hkv*G .. hkv*G+G-1); k, v: [N, d].
    Returns dQ [G, N, d], dK [N, d], dV [N, d] for the loss L = sum(O * dO).

    The pages say only that the backward recomputes S and P from Q, K, V
    ([YOLO11-FA2] section 2.3) and give no formulas, so this is the plain chain
    rule of the forward definition, on materialised S and P:
      dV_j  = sum_i P_ij dO_i
      dP_ij = <dO_i, v_j>
      dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
      dQ_i  = scale * sum_j dS_ij k_j
      dK_j  = scale * sum_i dS_ij q_i
    and, because K and V are shared by the G heads ([FA-GQA]
    repeat_interleave), dK and dV sum over those heads. Under dropout
    (``dropout`` = (p, seed, offset, bh0), head g being bh0 + g) the forward is
    O = Pd V with Pd = P * M / (1 - p) for the fixed keep mask M, so dV uses
    Pd and dP picks up the same factor M / (1 - p) before the softmax step.
    """
    q = np.asarray(q, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    G, N, d = q.shape
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for g in range(G):
        for r0 in range(0, N, chunk):
            r1 = min(N, r0 + chunk)
            qc = q[g, r0:r1]
            doc = do[g, r0:r1]
            _, _, _, P = ref_fwd_head(qc, k, v, scale, causal, row0=r0, return_sp=True, window=window)
            keep, p = _keep_rows(None if dropout is None else dropout[:3],
                                 0 if dropout is None else dropout[3] + g, r0, r1, N)
            dP = doc @ v.T
            dP = _dropped(dP, keep, p)
            row_term = (P * dP).sum(axis=1)
            dS = P * (dP - row_term[:, None])
            dQ[g, r0:r1] = scale * (dS @ k)
            dK += scale * (dS.T @ qc)
            dV += _dropped(P, keep, p).T @ doc
    return dQ, dK, dV


def ref_bwd(q, k, v, do, scale, causal=False, kv_heads=None, chunk=DEFAULT_CHUNK, window=None,
            dropout=None):
    """Backward for full [B, H, N, d] arrays; see :func:`ref_bwd_group`.

    ``kv_heads`` restricts the work to a list of (b, hkv) pairs (each brings its
    G query heads); other entries are left NaN.
    """
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    G = Hq // Hkv
    dQ = np.full((B, Hq, N, d), np.nan)
    dK = np.full((B, Hkv, N, d), np.nan)
    dV = np.full((B, Hkv, N, d), np.nan)
    if kv_heads is None:
        kv_heads = [(b, h) for b in range(B) for h in range(Hkv)]
    for b, hkv in kv_heads:
        sl = slice(hkv * G, hkv * G + G)
        drop = None if dropout is None else (*dropout, b * Hq + hkv * G)
        dq, dk, dv = ref_bwd_group(q[b, sl], k[b, hkv], v[b, hkv], do[b, sl],
                                   scale, causal, chunk, window, drop)
        dQ[b, sl] = dq
        dK[b, hkv] = dk
        dV[b, hkv] = dv
    return dQ, dK, dV


def blockwise_online_fwd(q, k, v, scale, causal=False, block_r=64, block_c=64, window=None):
    """The blockwise online-softmax forward of one head, in fp64.

    Follows the [CANN-FA] online-softmax pseudocode (section on online
    softmax) step by step, with the scale that the pseudocode leaves out put
    back on the scores before the maximum, and with the mask applied to the
    scores of each block:
      for each query block, for each key/value block:
        scores  = scale * Q_blk K_blk^T (masked)
        m_new   = max(m, row max of scores)
        corr    = exp(m - m_new);  O *= corr;  l *= corr
        P_blk   = exp(scores - m_new);  O += P_blk V_blk;  l += row sum P_blk
        m       = m_new
      O /= l
    Returns O [N, d] and LSE [N] = m + ln l. [YOLO11-FA2] section 2.2 and the
    same [CANN-FA] section state that this equals the plain softmax result up
    to floating-point summation order; the CPU tests check exactly that.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    O = np.zeros((N, d))
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    for i0 in range(0, N, block_r):
        i1 = min(N, i0 + block_r)
        for j0 in range(0, N, block_c):
            j1 = min(N, j0 + block_c)
            scores = (q[i0:i1] @ k[j0:j1].T) * scale
            if causal or window is not None:
                ii = np.arange(i0, i1)[:, None]
                jj = np.arange(j0, j1)[None, :]
                ok = jj <= ii
                if window is not None:
                    ok &= jj > ii - window
                scores = np.where(ok, scores, -np.inf)
            m_old = m[i0:i1]
            m_new = np.maximum(m_old, scores.max(axis=1))
            # exp(-inf - (-inf)) is undefined; a row whose keys have all been
            # masked so far has O = 0 and l = 0, so any finite factor is right.
            with np.errstate(invalid="ignore"):
                corr = np.where(np.isneginf(m_new), 1.0, np.exp(m_old - m_new))
                P_blk = np.where(np.isneginf(m_new)[:, None], 0.0,
                                 np.exp(scores - m_new[:, None]))
            O[i0:i1] *= corr[:, None]
            l[i0:i1] *= corr
            O[i0:i1] += P_blk @ v[j0:j1]
            l[i0:i1] += P_blk.sum(axis=1)
            m[i0:i1] = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(l[:, None] > 0, O / l[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return O, lse


def ref_decode(q, k, v, scale, causal=False, kv_lens=None, window=None):
    """Attention of Nq new queries per sequence against a key/value cache.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] caches whose first L_b rows are
    valid, L_b = kv_lens[b] clamped to [0, Nk] (all Nk rows when kv_lens is
    None). Returns (O [B, Hq, Nq, d], LSE [B, Hq, Nq]) in float64.

    The pages describe decoding only through the KV cache that GQA shrinks
    ([FA-GQA], sections on the KV cache of MHA and on GQA); they fix no
    alignment between the new queries and the cached keys. The reading taken:
    the cache already holds the keys of the new tokens, so query i sits at
    position p_i = L_b - Nq + i, and its allowed keys are the A_i of a
    sequence of length L_b at row p_i (all j < L_b; j <= p_i under the causal
    mask; p_i - W < j <= p_i under a window of W). Decoding is then exactly
    the last Nq rows of self-attention over the L_b cached positions. A query
    with no allowed key (p_i < 0, i.e. L_b < Nq, under a causal mask; or an
    empty cache) gets O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d]")
    B, Hq, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape}")
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        L = Nk if kv_lens is None else int(min(max(int(kv_lens[b]), 0), Nk))
        if L == 0:
            continue
        for hq in range(Hq):
            hkv = kv_head_of(hq, Hq, Hkv)
            o, lse = ref_fwd_head(q[b, hq], k[b, hkv, :L], v[b, hkv, :L], scale, causal,
                                  row0=L - Nq, window=window)
            O[b, hq] = o
            LSE[b, hq] = lse
    return O, LSE
