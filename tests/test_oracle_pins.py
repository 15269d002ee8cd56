"""The fp64 oracle against brute force, hand-worked cases, closed forms,
invariants and finite differences (CPU only)."""

import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def fwd(q, k, v, scale, causal):
    return oracle.ref_fwd(q, k, v, scale, causal, chunk=4)


def bwd(q, k, v, do, scale, causal):
    return oracle.ref_bwd(q, k, v, do, scale, causal, chunk=4)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (1, 2, 1, 5, 3), (2, 4, 2, 6, 4), (1, 3, 3, 4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(shape, causal):
    pins.check_brute_force(fwd, 100 + sum(shape), *shape, causal)


def test_hand_2x2_forward():
    pins.check_hand_2x2_fwd(fwd)


def test_hand_2x2_backward():
    pins.check_hand_2x2_bwd(bwd)


@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(causal):
    pins.check_zero_queries(fwd, causal)
    pins.check_library_softmax(fwd, causal)


def test_special_cases():
    pins.check_causal_first_row(fwd)
    pins.check_single_key(fwd)
    pins.check_identical_keys(fwd)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    pins.check_key_shift(fwd, causal)
    pins.check_value_shift(fwd, causal)
    pins.check_convex_hull(fwd, causal)
    pins.check_rows_sum_to_one(oracle.ref_fwd_head, causal)


def test_key_permutation():
    pins.check_key_permutation(fwd)


@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(G, causal):
    pins.check_gqa_is_repeated_mha(fwd, bwd, G, causal=causal)


def test_mqa_equals_repeated_mha():
    pins.check_gqa_is_repeated_mha(fwd, bwd, 6, Hkv=1)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    pins.check_bwd_identities(bwd, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 3), (1, 2, 2, 4, 2)])
def test_finite_differences(causal, shape):
    pins.check_finite_differences(fwd, bwd, causal, 200 + sum(shape), *shape)


@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_online_equals_definition(causal):
    pins.check_blockwise_equals_plain(oracle.blockwise_online_fwd, oracle.ref_fwd_head, causal)


@pytest.mark.parametrize("chunk", [1, 3, 64, 1000])
def test_row_chunking_is_exact(chunk):
    q, k, v, do = pins.rng_arrays(30, 1, 2, 1, 37, 8)
    O, L = oracle.ref_fwd(q, k, v, 0.3, True, chunk=1000)
    O2, L2 = oracle.ref_fwd(q, k, v, 0.3, True, chunk=chunk)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(L2, L, atol=1e-14)
    g = oracle.ref_bwd(q, k, v, do, 0.3, True, chunk=1000)
    g2 = oracle.ref_bwd(q, k, v, do, 0.3, True, chunk=chunk)
    for a, b in zip(g, g2):
        np.testing.assert_allclose(b, a, atol=1e-13)


def test_head_subsets_match_full():
    q, k, v, do = pins.rng_arrays(31, 2, 4, 2, 9, 4)
    O, L = oracle.ref_fwd(q, k, v, 0.5, True)
    Os, Ls = oracle.ref_fwd(q, k, v, 0.5, True, heads=[(1, 3)])
    np.testing.assert_array_equal(Os[1, 3], O[1, 3])
    assert np.isnan(Os[0, 0]).all()
    g = oracle.ref_bwd(q, k, v, do, 0.5, True)
    gs = oracle.ref_bwd(q, k, v, do, 0.5, True, kv_heads=[(0, 1)])
    np.testing.assert_array_equal(gs[0][0, 2:4], g[0][0, 2:4])
    np.testing.assert_array_equal(gs[1][0, 1], g[1][0, 1])
    np.testing.assert_array_equal(gs[2][0, 1], g[2][0, 1])


def test_rejects_bad_grouping():
    q, k, v, _ = pins.rng_arrays(32, 1, 3, 2, 4, 2, with_do=False)
    with pytest.raises(ValueError):
        oracle.ref_fwd(q, k, v, 1.0)
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 3, 2)


def fwd_w(q, k, v, scale, window):
    return oracle.ref_fwd(q, k, v, scale, True, chunk=4, window=window)


def bwd_w(q, k, v, do, scale, window):
    return oracle.ref_bwd(q, k, v, do, scale, True, chunk=4, window=window)


@pytest.mark.parametrize("shape,window", [((1, 2, 1, 6, 3), 1), ((2, 4, 2, 6, 4), 2), ((1, 3, 3, 7, 2), 4)])
def test_window_brute_force(shape, window):
    pins.check_window_brute_force(fwd_w, 300 + window, *shape, window)


def test_window_special_cases():
    pins.check_window_special_cases(fwd, fwd_w)


def test_window_blockwise_online():
    pins.check_window_blockwise(oracle.blockwise_online_fwd, oracle.ref_fwd_head)


def test_window_gradients():
    pins.check_window_gradients(fwd_w, bwd_w)


def test_window_rejects_zero():
    with pytest.raises(ValueError):
        oracle.allowed_mask(0, 3, 3, True, 0)


# ------------------------------------------------------------------- decoding

def dec(q, k, v, scale, causal, kv_lens, window):
    return oracle.ref_decode(q, k, v, scale, causal, kv_lens=kv_lens, window=window)


def fwd_full(q, k, v, scale, causal, window):
    return oracle.ref_fwd(q, k, v, scale, causal, chunk=3, window=window)


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 3), (True, 1)])
def test_decode_brute_force(causal, window):
    pins.check_decode_brute_force(dec, 40 + (window or 0), causal, window)


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 4), (True, 20)])
def test_decode_is_last_rows_of_self_attention(causal, window):
    pins.check_decode_is_last_rows(dec, fwd_full, causal, window)


def test_decode_special_cases():
    pins.check_decode_special_cases(dec)


# ------------------------------------------------------------ Philox, dropout

from oracle import philox as ph  # noqa: E402


def fwd_d(q, k, v, scale, causal, drop):
    return oracle.ref_fwd(q, k, v, scale, causal, chunk=4, dropout=drop)


def bwd_d(q, k, v, do, scale, causal, drop):
    return oracle.ref_bwd(q, k, v, do, scale, causal, chunk=4, dropout=drop)


def test_philox_matches_numpy_philox4x64():
    pins.check_philox_against_numpy(ph.philox)


def test_philox_weyl_constants():
    pins.check_philox_weyl_constants(ph.CONSTANTS)


def _run_rocrand(cases):
    """Builds tests/rocrand_philox.cpp (rocRAND's Philox engine, host code)
    and runs it on the cases."""
    import shutil
    import subprocess
    import tempfile
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("no ROCm toolchain with rocRAND headers")
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox.cpp")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "rocrand_philox")
        subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, capture_output=True)
        inp = "".join(f"{a} {b} {c}\n" for a, b, c in cases)
        out = subprocess.run([exe], input=inp, check=True, capture_output=True, text=True).stdout
    return [[int(w, 16) for w in line.split()] for line in out.splitlines()]


def test_philox32_matches_rocrand():
    pins.check_philox32_against_rocrand(ph.philox4x32, _run_rocrand)


def test_philox32_stream():
    pins.check_philox32_stream(ph.philox, ph.philox4x32)


def test_keep_mask():
    pins.check_keep_mask(ph.dropout_keep, ph.keep_threshold)


def test_dropout_forward():
    pins.check_dropout_forward(fwd_d, lambda q, k, v, s, c: oracle.ref_fwd(q, k, v, s, c, chunk=4),
                               ph.dropout_keep)


def test_dropout_expectation():
    pins.check_dropout_expectation(fwd_d, lambda q, k, v, s, c: oracle.ref_fwd(q, k, v, s, c, chunk=4))


def test_dropout_gradients():
    pins.check_dropout_gradients(fwd_d, bwd_d)
