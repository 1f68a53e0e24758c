"""Pins of the chunk-score oracle (token log-probabilities and s = s_I + s_P)
to values the mathematics fixes: closed forms, a library routine, invariants
and hand-built cases whose scores are known exactly."""
import math

import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
import synth


def test_uniform_logits_give_minus_log_vocab():
    """Equal logits: every token has probability 1/V."""
    for v in (1, 2, 7, 1000, 152064):
        z = np.full((3, v), 0.625, dtype=np.float32)
        lp = oracle.token_log_probs(z, np.array([0, v // 2, v - 1]))
        assert np.allclose(lp, -math.log(v), rtol=0, atol=1e-12)


def test_two_token_closed_form():
    """V = 2: log p(0) = -ln(1 + e^(b - a))."""
    rng = np.random.default_rng(5)
    ab = rng.normal(0, 4, size=(50, 2)).astype(np.float32)
    lp = oracle.token_log_probs(ab, np.zeros(50, dtype=np.int32))
    a, b = ab[:, 0].astype(np.float64), ab[:, 1].astype(np.float64)
    assert np.allclose(lp, -np.log1p(np.exp(b - a)), rtol=0, atol=1e-12)


def test_matches_library_log_softmax():
    rng = np.random.default_rng(6)
    z = (rng.normal(0, 3, size=(20, 4099))).astype(np.float32)
    t = rng.integers(0, 4099, size=20)
    want = log_softmax(z.astype(np.float64), axis=1)[np.arange(20), t]
    assert np.allclose(oracle.token_log_probs(z, t), want, rtol=0, atol=1e-11)


def test_bf16_bits_decode_exactly():
    """bf16 logits are read as the exact values their bits encode."""
    rng = np.random.default_rng(7)
    z = rng.normal(0, 2, size=(4, 300)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(z)
    exact = (bits.astype(np.uint32) << 16).view(np.float32)
    t = np.array([3, 0, 299, 150])
    assert np.array_equal(oracle.token_log_probs(bits, t), oracle.token_log_probs(exact, t))


def test_shift_invariance_and_dominant_target():
    rng = np.random.default_rng(8)
    z = rng.normal(0, 1, size=(5, 777)).astype(np.float64)
    t = rng.integers(0, 777, size=5)
    assert np.allclose(oracle.token_log_probs(z + 37.5, t), oracle.token_log_probs(z, t), rtol=0, atol=1e-11)
    big = z.copy()
    big[np.arange(5), t] = 1.0e4            # the target takes all the mass
    assert np.all(np.abs(oracle.token_log_probs(big, t)) <= 1e-300)


def test_chunk_score_signs_and_rows():
    """Chunk 0: query rows uniform (s_I = n_q ln V), pseudo rows certain
    (s_P = 0).  Chunk 1: query rows certain (s_I = 0), pseudo rows uniform
    (s_P = -n_p ln V).  This pins the sign of each part and which rows feed
    which part."""
    v, n_q, n_p = 50, 3, 4
    logits = np.zeros((2, n_q + n_p, v))
    target = np.tile(np.arange(n_q + n_p) % v, (2, 1))
    logits[0, n_q:, :] = -1.0e4
    logits[0, np.arange(n_q, n_q + n_p), target[0, n_q:]] = 0.0
    logits[1, :n_q, :] = -1.0e4
    logits[1, np.arange(n_q), target[1, :n_q]] = 0.0
    s_i, s_p, s = oracle.chunk_scores(logits, target, n_q, n_p)
    assert np.allclose(s_i, [n_q * math.log(v), 0.0], rtol=0, atol=1e-12)
    assert np.allclose(s_p, [0.0, -n_p * math.log(v)], rtol=0, atol=1e-12)
    assert np.array_equal(s, s_i + s_p)


@pytest.mark.parametrize("n_q,n_p", [(4, 0), (0, 5), (3, 6)])
def test_chunk_score_is_sum_of_row_log_probs(n_q, n_p):
    """s_I and s_P are the plain sums of the per-row values of the library
    log-softmax, taken on each chunk's own rows."""
    rng = np.random.default_rng(9)
    n_c, v = 3, 513
    z = rng.normal(0, 2, size=(n_c, n_q + n_p, v))
    t = rng.integers(0, v, size=(n_c, n_q + n_p))
    lp = log_softmax(z, axis=2)[np.arange(n_c)[:, None], np.arange(n_q + n_p)[None, :], t]
    s_i, s_p, s = oracle.chunk_scores(z, t, n_q, n_p)
    assert np.allclose(s_i, -lp[:, :n_q].sum(axis=1), rtol=0, atol=1e-10)
    assert np.allclose(s_p, lp[:, n_q:].sum(axis=1), rtol=0, atol=1e-10)
    if n_p == 0:
        assert np.all(s_i > 0) and np.all(s_p == 0)       # an NLL is positive
    if n_q == 0:
        assert np.all(s_p < 0) and np.all(s_i == 0)       # a log-likelihood is negative
