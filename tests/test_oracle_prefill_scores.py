"""Pins of the oracle's prefill token weights and initial window scores (CPU):
rows of a causal softmax sum to one (so every head's weights sum to T), equal
keys give harmonic-number weights in closed form, a scalar brute force on tiny
inputs, and the window sums.  The blocked one-head form (for long prefills)
is pinned by the same closed form across block edges and by the full form."""
import math

import numpy as np
import pytest

from oracle.prefill_scores import head_token_weights, token_weights, window_scores


def test_weights_of_each_head_sum_to_the_number_of_queries():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((6, 37, 16)) * 2
    k = rng.standard_normal((2, 37, 16)) * 2
    w = token_weights(q, k)
    assert w.shape == (6, 37)
    np.testing.assert_allclose(w.sum(axis=1), 37.0, rtol=1e-12)
    assert (w > 0).all()


def test_equal_keys_give_harmonic_weights():
    """All keys equal: query tau spreads 1/(tau+1) over keys 0..tau, so
    w_t = sum_{tau=t}^{T-1} 1/(tau+1) = H_T - H_t."""
    T = 50
    q = np.random.default_rng(2).standard_normal((4, T, 8))
    k = np.tile(np.random.default_rng(3).standard_normal((1, 1, 8)), (1, T, 1))
    w = token_weights(q, k)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    want = H[T] - H[np.arange(T)]
    for h in range(4):
        np.testing.assert_allclose(w[h], want, rtol=1e-12)


def test_scalar_brute_force():
    rng = np.random.default_rng(4)
    hq, hkv, T, D = 4, 2, 9, 4
    q = rng.standard_normal((hq, T, D))
    k = rng.standard_normal((hkv, T, D))
    got = token_weights(q, k)
    for h in range(hq):
        want = [0.0] * T
        for tau in range(T):
            z = [sum(q[h, tau, d] * k[h // 2, t, d] for d in range(D)) / math.sqrt(D) for t in range(tau + 1)]
            mx = max(z)
            e = [math.exp(x - mx) for x in z]
            s = sum(e)
            for t in range(tau + 1):
                want[t] += e[t] / s
        np.testing.assert_allclose(got[h], want, rtol=1e-12)


def test_window_sums_cover_every_token_once():
    rng = np.random.default_rng(5)
    w = rng.random((3, 21))
    s = window_scores(w, 8)
    assert s.shape == (3,)
    np.testing.assert_allclose(s, [w[:, 0:8].sum(), w[:, 8:16].sum(), w[:, 16:21].sum()], rtol=1e-14)
    assert s.sum() == pytest.approx(w.sum(), rel=1e-14)


def test_blocked_head_weights_equal_the_full_form():
    """Blocks of query rows that do and do not divide T, and a block longer
    than T, give the full form's weights for every head."""
    rng = np.random.default_rng(6)
    hq, hkv, T, D = 4, 2, 53, 16
    q = rng.standard_normal((hq, T, D)) * 2
    k = rng.standard_normal((hkv, T, D)) * 2
    full = token_weights(q, k)
    for block in (1, 7, 16, 53, 64):
        for h in range(hq):
            np.testing.assert_allclose(head_token_weights(q[h], k[h // 2], block), full[h], rtol=1e-12)


def test_blocked_head_weights_harmonic_across_blocks():
    """Equal keys: w_t = H_T - H_t, over 5000 tokens in blocks of 1024 (the
    last block partial); the weights sum to T."""
    T = 5000
    q = np.random.default_rng(7).standard_normal((T, 8))
    k = np.tile(np.random.default_rng(8).standard_normal((1, 8)), (T, 1))
    w = head_token_weights(q, k, 1024)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    np.testing.assert_allclose(w, H[T] - H[np.arange(T)], rtol=1e-11)
    assert w.sum() == pytest.approx(T, rel=1e-12)
