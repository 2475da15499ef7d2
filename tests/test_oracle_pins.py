"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins
from synth_inputs import to_f64


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_cached_equals_recompute_all_dtypes(dtype):
    pins.check_cached_equals_recompute(dtype=dtype)


def test_probabilities_sum_to_one_directly():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 40, 8)) * 4
    k = rng.standard_normal((1, 2, 40, 8)) * 4
    _, p = oracle.naive_causal(q, k, rng.standard_normal((1, 2, 40, 8)), 0.5, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-13)
    assert (np.triu(p[0, 0], 1) == 0).all()


def test_cache_model_rejects_bad_state():
    c = oracle.CacheModel(1, 2, 1, 4, 3, np.float16)
    with pytest.raises(RuntimeError):
        c.prefill(0, np.zeros((2, 1, 4, 4), np.float16), np.zeros((2, 1, 4, 4), np.float16))
    c.prefill(0, np.zeros((2, 1, 2, 4), np.float16), np.zeros((2, 1, 2, 4), np.float16))
    with pytest.raises(RuntimeError):
        c.prefill(0, np.zeros((2, 1, 1, 4), np.float16), np.zeros((2, 1, 1, 4), np.float16))
    c.append(0, np.ones((2, 1, 1, 4), np.float16), np.ones((2, 1, 1, 4), np.float16))
    with pytest.raises(RuntimeError):
        c.append(0, np.ones((2, 1, 1, 4), np.float16), np.ones((2, 1, 1, 4), np.float16))
    assert (c.k[0, :, 0, 2] == 1).all() and (c.lengths[0] == 3).all()


def test_decode_heavy_rows_finite_and_matches_brute():
    # scores near +-45 (the x8 heavy keys) in a half-precision layout stay finite
    from synth_inputs import round_to
    rng = np.random.default_rng(5)
    L, D = 50, 16
    K = to_f64(round_to(rng.standard_normal((L, D)), "f16"), "f16")
    K[[3, 17, 40]] *= 8.0
    V = to_f64(round_to(rng.standard_normal((L, D)), "f16"), "f16")
    q = to_f64(round_to(rng.standard_normal(D), "f16"), "f16") * 2
    got = oracle.attend_row(q, K, V, 0.25)
    ref = np.array(oracle.brute([[[list(q)] * L]], [[K.tolist()]], [[V.tolist()]], 0.25))[0, 0, L - 1]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
