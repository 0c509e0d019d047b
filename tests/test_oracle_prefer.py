"""Pins for the oracle's dense-preference score (TailorKV article, section 2.1:
P = n_q - sum of the top-k attention probabilities of the last n_q queries,
quantization-friendly when P exceeds tau = 0.2).  CPU only."""
import numpy as np
import pytest

from oracle import attend as A
from oracle import select as S


def _probs(logits):
    z = np.asarray(logits, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def test_uniform_row_closed_form():
    for n, k in [(10, 3), (4096, 128), (7, 7), (5, 9), (6, 0)]:
        assert S.topk_mass(_probs(np.zeros(n)), k) == pytest.approx(min(k, n) / n, abs=1e-15)


def test_dominant_token_and_two_level_closed_form():
    """k tokens at logit L and n - k at 0: mass = k e^L / (k e^L + n - k)."""
    n, k, L = 1000, 40, 5.0
    z = np.zeros(n)
    z[np.random.default_rng(1).choice(n, k, replace=False)] = L
    want = k * np.exp(L) / (k * np.exp(L) + (n - k))
    assert S.topk_mass(_probs(z), k) == pytest.approx(want, rel=1e-13)
    # asking for fewer takes the high ones only; more adds low ones at e^0 each
    assert S.topk_mass(_probs(z), 10) == pytest.approx(10 * np.exp(L) / (k * np.exp(L) + n - k), rel=1e-13)
    assert S.topk_mass(_probs(z), 50) == pytest.approx((k * np.exp(L) + 10) / (k * np.exp(L) + n - k), rel=1e-13)


def test_brute_force_and_ties():
    rng = np.random.default_rng(2)
    for _ in range(30):
        n = int(rng.integers(1, 300))
        z = rng.integers(-3, 3, size=n).astype(np.float64)   # many ties
        p = _probs(z)
        k = int(rng.integers(0, n + 3))
        brute = sum(sorted(p.tolist(), reverse=True)[:k])
        assert S.topk_mass(p, k) == pytest.approx(brute, rel=1e-14, abs=1e-16)
        # the mass is at most 1 and grows with k
        assert S.topk_mass(p, k) <= 1 + 1e-15
        if k:
            assert S.topk_mass(p, k) >= S.topk_mass(p, k - 1)


def test_mass_from_attention_rows_and_decision():
    """The probabilities are exp(logit - lse) of the oracle's attention rows."""
    rng = np.random.default_rng(3)
    q = rng.normal(size=(4, 128)).astype(np.float16)
    k = rng.normal(size=(500, 128))
    v = rng.normal(size=(500, 128))
    sm = float(np.float32(1 / np.sqrt(128)))
    _, lse, logits = A.attend_group(q, k, v, sm)
    for h in range(4):
        p = np.exp(logits[h] - lse[h])
        assert p.sum() == pytest.approx(1.0, abs=1e-12)
        assert S.topk_mass(p, 500) == pytest.approx(1.0, abs=1e-12)
    # the page's two layers: 0.7178 (dense layer 0) and 0.0473 (layer 16) with tau 0.2
    assert S.quantization_friendly(0.7178) and not S.quantization_friendly(0.0473)
    assert S.dense_preference([0.25, 0.5]) == pytest.approx(1.25)
