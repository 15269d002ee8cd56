"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a one-spot text edit of ``oracle/attention.py`` (a dropped term,
a wrong sign or index, a transposed operand, a wrong mask), loaded as a
separate module on the CPU. The pin suite of ``tests/oracle_pins.py`` is run
against it and is expected to reject it.
"""

import importlib.util
import os
import types

import pytest

from oracle import philox
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "attention.py")

MUTANTS = {
    "scale_dropped": ("S = (q @ k.T) * scale", "S = (q @ k.T)"),
    "gqa_modulo_mapping": ("return hq // (Hq // Hkv)", "return hq % Hkv"),
    "causal_excludes_diagonal": ("ok = j <= i", "ok = j < i"),
    "causal_transposed": ("ok = j <= i", "ok = j >= i"),
    "lse_without_max": ("safe_m + np.log(den)", "np.log(den)"),
    "softmax_not_normalised": ("E / den[:, None]", "E"),
    "pv_transposed": ("O = _dropped(P, keep, p_drop) @ v", "O = P.T @ v[: P.shape[0]]"),
    "row_term_dropped": ("dS = P * (dP - row_term[:, None])", "dS = P * dP"),
    "row_term_sign": ("dS = P * (dP - row_term[:, None])", "dS = P * (dP + row_term[:, None])"),
    "dk_scale_dropped": ("dK += scale * (dS.T @ qc)", "dK += (dS.T @ qc)"),
    "dq_sign": ("dQ[g, r0:r1] = scale * (dS @ k)", "dQ[g, r0:r1] = -scale * (dS @ k)"),
    "dv_uses_scores": ("dV += _dropped(P, keep, p).T @ doc",
                       "dV += np.where(np.isfinite(_s), _s, 0).T @ doc"),
    "dk_not_group_summed": ("dK += scale * (dS.T @ qc)", "dK = scale * (dS.T @ qc) if g == G - 1 else dK"),
    "dp_transposed_v": ("dP = doc @ v.T", "dP = doc @ v[::-1].T"),
    "online_l_not_rescaled": ("l[i0:i1] *= corr", "pass"),
    "online_o_not_rescaled": ("O[i0:i1] *= corr[:, None]", "pass"),
    "online_uses_old_max": ("np.exp(scores - m_new[:, None])",
                            "np.exp(scores - np.where(np.isfinite(m_old), m_old, m_new)[:, None])"),
    "online_drops_lse_max": ("m + np.log(l)", "np.log(l)"),
    "window_off_by_one": ("ok &= j > i - window", "ok &= j >= i - window"),
    "window_ignored": ("ok &= j > i - window", "pass"),
    "decode_top_left_alignment": ("row0=L - Nq, window=window)", "row0=0, window=window)"),
    "decode_alignment_off_by_one": ("row0=L - Nq, window=window)", "row0=L - Nq + 1, window=window)"),
    "decode_ignores_lengths": ("L = Nk if kv_lens is None else", "L = Nk if True else"),
    "decode_length_not_clamped": ("int(min(max(int(kv_lens[b]), 0), Nk))", "int(kv_lens[b])"),
    "dropout_not_rescaled": ("np.where(keep, P / (1.0 - p_drop), 0.0)", "np.where(keep, P, 0.0)"),
    "dropout_mask_not_on_dP": ("dP = _dropped(dP, keep, p)", "dP = dP"),
    "dropout_dv_undropped": ("dV += _dropped(P, keep, p).T @ doc", "dV += P.T @ doc"),
    "dropout_bwd_same_mask_for_group": ("dropout[3] + g, r0, r1, N)", "dropout[3], r0, r1, N)"),
    "dropout_fwd_head_index_without_batch": ("_keep_rows(dropout, b * Hq + hq,", "_keep_rows(dropout, hq,"),
}


def load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    src = src.replace(old, new)
    if "_s" in new:
        src = src.replace("_, _, _, P = ref_fwd_head(", "_, _, _s, P = ref_fwd_head(")
    mod = types.ModuleType("oracle_mutant")
    mod.__package__ = "oracle"  # the copy imports the oracle's Philox module relatively
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def run_all_pins(mod):
    fwd = lambda q, k, v, s, c: mod.ref_fwd(q, k, v, s, c, chunk=4)
    bwd = lambda q, k, v, do, s, c: mod.ref_bwd(q, k, v, do, s, c, chunk=4)
    pins.all_forward_checks(fwd)
    pins.all_backward_checks(fwd, bwd)
    for causal in (False, True):
        pins.check_rows_sum_to_one(mod.ref_fwd_head, causal)
        pins.check_blockwise_equals_plain(mod.blockwise_online_fwd, mod.ref_fwd_head, causal)
    fwd_w = lambda q, k, v, s, w: mod.ref_fwd(q, k, v, s, True, chunk=4, window=w)
    bwd_w = lambda q, k, v, do, s, w: mod.ref_bwd(q, k, v, do, s, True, chunk=4, window=w)
    pins.check_window_brute_force(fwd_w, 301, 1, 2, 1, 6, 3, 2)
    pins.check_window_special_cases(fwd, fwd_w)
    pins.check_window_gradients(fwd_w, bwd_w)
    dec = lambda q, k, v, s, c, lens, w: mod.ref_decode(q, k, v, s, c, kv_lens=lens, window=w)
    full = lambda q, k, v, s, c, w: mod.ref_fwd(q, k, v, s, c, chunk=3, window=w)
    for causal, window in ((False, None), (True, None), (True, 3)):
        pins.check_decode_brute_force(dec, 41, causal, window)
        pins.check_decode_is_last_rows(dec, full, causal, window)
    pins.check_decode_special_cases(dec)
    fwd_d = lambda q, k, v, s, c, drop: mod.ref_fwd(q, k, v, s, c, chunk=4, dropout=drop)
    bwd_d = lambda q, k, v, do, s, c, drop: mod.ref_bwd(q, k, v, do, s, c, chunk=4, dropout=drop)
    pins.check_dropout_forward(fwd_d, fwd, philox.dropout_keep)
    pins.check_dropout_gradients(fwd_d, bwd_d)


def test_unmutated_copy_passes():
    run_all_pins(load_mutant("DEFAULT_CHUNK = 1024", "DEFAULT_CHUNK = 1024"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = load_mutant(*MUTANTS[name])
    with pytest.raises(Exception):
        run_all_pins(mod)


# Planted mistakes in a copy of oracle/philox.py (the dropout stream), each
# rejected by the stream pins.
PHILOX_SRC = os.path.join(os.path.dirname(SRC), "philox.py")
PHILOX_MUTANTS = {
    "both_keys_same_half": ("(16 * (j % 2))", "(16 * (j % 1))"),
    "row_word_from_key": ("np.choose((i % 4) * np.ones_like(j), words)", "np.choose((j % 4) * np.ones_like(i), words)"),
    "threshold_32_bit": ("np.float64(p) * 65536.0)), 65535)", "np.float64(p) * 4294967296.0)), 4294967295)"),
    "multiplier_bit_flip": ("32: dict(M0=0xD2511F53,", "32: dict(M0=0xD2511F57,"),
    "weyl_constant_off_by_one": ("W0=0x9E3779B9, W1=0xBB67AE85", "W0=0x9E3779B9, W1=0xBB67AE86"),
    "hi_lo_swapped": ("c = [(p1 >> s32) ^ c[1] ^ k0, p1 & m32, (p0 >> s32) ^ c[3] ^ k1, p0 & m32]",
                      "c = [(p1 & m32) ^ c[1] ^ k0, p1 >> s32, (p0 >> s32) ^ c[3] ^ k1, p0 & m32]"),
}


def load_philox_mutant(old, new):
    src = open(PHILOX_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("philox_mutant")
    exec(compile(src.replace(old, new), "philox_mutant", "exec"), mod.__dict__)
    return mod


def run_stream_pins(mod):
    pins.check_keep_mask(mod.dropout_keep, mod.keep_threshold)
    pins.check_philox_weyl_constants(mod.CONSTANTS)
    pins.check_philox32_against_rocrand(mod.philox4x32, _rocrand_cases)


_ROCRAND_CACHE = {}


def _rocrand_cases(cases):
    key = tuple(cases)
    if key not in _ROCRAND_CACHE:
        from tests.test_oracle_pins import _run_rocrand
        _ROCRAND_CACHE[key] = _run_rocrand(cases)
    return _ROCRAND_CACHE[key]


def test_unmutated_philox_passes():
    run_stream_pins(load_philox_mutant("def effective_p(", "def effective_p("))


@pytest.mark.parametrize("name", sorted(PHILOX_MUTANTS))
def test_philox_mutant_is_caught(name):
    mod = load_philox_mutant(*PHILOX_MUTANTS[name])
    with pytest.raises(Exception):
        run_stream_pins(mod)
