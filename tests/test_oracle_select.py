"""Pins for the oracle's scoring and Top-K selection (CPU only)."""
import numpy as np
import pytest

from oracle import select as S


def test_critical_channels_hand_example():
    """s_c = max_h |q_{h,c}| * max|K_c| (TailorKV 2.3), top-n ascending, ties to the lower channel."""
    q = np.zeros((2, 128), np.float16)
    kabs = np.ones(128, np.float16)
    q[0, 5] = -3.0      # s = 3
    q[1, 9] = 2.0       # s = 2 * 4 = 8
    kabs[9] = 4.0
    q[0, 70] = 1.0      # s = 1 * 8 = 8  (ties channel 9: 9 wins)
    kabs[70] = 8.0
    q[1, 100] = -0.5    # s = 0.5 * 10 = 5
    kabs[100] = 10.0
    assert S.critical_channels(q, kabs, 1).tolist() == [9]
    assert S.critical_channels(q, kabs, 2).tolist() == [9, 70]
    assert S.critical_channels(q, kabs, 4).tolist() == [5, 9, 70, 100]
    assert S.critical_channels(q, kabs, 500).tolist() == list(range(128))


def test_critical_channels_brute_force_and_permutation():
    rng = np.random.default_rng(21)
    for _ in range(50):
        q = rng.normal(size=(4, 128)).astype(np.float16)
        kabs = np.abs(rng.normal(size=128) * 3).astype(np.float16)
        # plant some exact ties
        kabs[::17] = kabs[0]
        q[:, ::17] = q[:, :1]
        s = [max(abs(float(q[h, c])) for h in range(4)) * float(kabs[c]) for c in range(128)]
        brute = sorted(sorted(range(128), key=lambda c: (-s[c], c))[:8])
        got = S.critical_channels(q, kabs, 8)
        assert got.tolist() == brute
        perm = rng.permutation(128)
        gotp = S.critical_channels(q[:, perm], kabs[perm], 8)
        # permuting channels permutes the choice (up to tie order, absent here after the check)
        if len(set(s[c] for c in brute)) == 8 and sorted(s)[-9] < min(s[c] for c in brute):
            assert sorted(perm[gotp].tolist()) == brute


def test_scores_closed_forms():
    rng = np.random.default_rng(22)
    keys = rng.integers(-50, 50, size=(40, 128)).astype(np.float64)
    # unit query picks one channel
    q = np.zeros((1, 128), np.float16)
    q[0, 17] = 1.0
    assert np.array_equal(S.token_scores(q, keys, range(128)), keys[:, 17])
    q[0, 17] = -1.0
    assert np.array_equal(S.token_scores(q, keys, range(128)), -keys[:, 17] + 0.0)
    # all-ones query on integer keys: exact integer row sums
    q1 = np.ones((1, 128), np.float16)
    assert S.token_scores(q1, keys, range(128)).tolist() == [float(sum(int(x) for x in row)) for row in keys]
    # GQA: max over the group's heads
    q2 = np.zeros((2, 128), np.float16)
    q2[0, 3] = 1.0
    q2[1, 4] = 1.0
    assert np.array_equal(S.token_scores(q2, keys, range(128)), np.maximum(keys[:, 3], keys[:, 4]))
    # only the listed channels count
    assert np.array_equal(S.token_scores(q1, keys, [2, 5]), keys[:, 2] + keys[:, 5])
    # a zero query gives +0.0, never -0.0
    z = S.token_scores(np.zeros((1, 128), np.float16), -np.abs(keys), range(128))
    assert np.all(z == 0) and not np.any(np.signbit(z))


def test_critical_with_every_channel_is_exact_score():
    rng = np.random.default_rng(23)
    q = rng.normal(size=(4, 128)).astype(np.float16)
    keys = rng.normal(size=(300, 128)).astype(np.float16).astype(np.float64)
    kabs = np.abs(keys).max(axis=0).astype(np.float16)
    ch = S.critical_channels(q, kabs, 128)
    assert np.array_equal(S.token_scores(q, keys, ch), S.token_scores(q, keys, np.arange(128)))


def test_scores_match_exact_rational_sums_on_fp16_data():
    """fp16 x fp16 products are exact in fp64 and, at these magnitudes, so is the sum."""
    from fractions import Fraction
    rng = np.random.default_rng(24)
    q = rng.normal(size=(1, 128)).astype(np.float16)
    keys = rng.normal(size=(20, 128)).astype(np.float16)
    got = S.token_scores(q, keys.astype(np.float64), range(128))
    for t in range(20):
        exact = sum(Fraction(float(q[0, c])) * Fraction(float(keys[t, c])) for c in range(128))
        assert got[t] == float(exact)


def _brute_topk(r, lo, hi, k):
    cand = [t for t in range(lo, hi)]
    best = sorted(cand, key=lambda t: (-r[t], t))[: max(k, 0)]
    return sorted(best)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 300))
    r = rng.integers(0, 12, size=n).astype(np.float64)   # many exact ties
    r[rng.integers(0, n)] = -0.0 + 0.0
    for k in [0, 1, n - 1, n, n + 5, int(rng.integers(0, n + 1))]:
        for lo, hi in [(0, n), (min(4, n), max(n - 7, 0)), (3, 2)]:
            got = S.topk_indices(r, lo, hi, k, k_max=n + 8)
            want = _brute_topk(r, max(lo, 0), min(hi, n), k)
            assert got[: len(want)].tolist() == want
            assert np.all(got[len(want):] == -1)


def test_topk_selected_dominate_unselected():
    rng = np.random.default_rng(31)
    r = rng.normal(size=5000)
    sel = S.topk_indices(r, 10, 4900, 300, 300)
    mask = np.zeros(5000, bool)
    mask[sel] = True
    cand = np.zeros(5000, bool)
    cand[10:4900] = True
    assert r[mask].min() >= r[cand & ~mask].max()
    assert np.all(np.diff(sel) > 0)


def test_attended_tokens_hand_example():
    assert S.attended_tokens("drop", 10, 2, 3, [4, 6, -1]).tolist() == [0, 1, 4, 6, 7, 8, 9]
    # selected ids inside the sink or window ranges are not double counted
    assert S.attended_tokens("drop", 10, 2, 3, [1, 8]).tolist() == [0, 1, 7, 8, 9]
    # sinks and window overlapping on a short sequence
    assert S.attended_tokens("drop", 4, 2, 3, []).tolist() == [0, 1, 2, 3]
    assert S.attended_tokens("dense", 5, 2, 3, [1]).tolist() == [0, 1, 2, 3, 4]
    assert S.keep_set(10, 2, 3, [4]).tolist() == [1, 1, 0, 0, 1, 0, 0, 1, 1, 1]


def test_topk_output_capacity_caps_k():
    r = np.arange(50, dtype=np.float64)
    got = S.topk_indices(r, 0, 50, 40, 8)
    assert got.tolist() == list(range(42, 50))
