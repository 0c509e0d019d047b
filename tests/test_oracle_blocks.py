"""Pins for the oracle's block-granular selection (meeting-LLM article, part 2
section 1.1 and section 8.1: mean importance per block, top blocks kept).  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import attend as A
from oracle import select as S
from oracle import step as ST


def test_block_range_hand_examples():
    assert S.block_range(4096, 4, 64) == (1, 63)      # blocks 1..62 lie inside [4, 4032)
    assert S.block_range(4096, 0, 0) == (0, 64)
    assert S.block_range(4097, 0, 0) == (0, 64)       # the incomplete block is not a candidate
    assert S.block_range(130, 64, 2) == (1, 2)        # [64, 128) only
    assert S.block_range(100, 4, 64) == (1, 1)        # no candidate
    assert S.block_range(0, 0, 0) == (0, 0)


def test_block_means_are_exact_on_integer_scores():
    """Integer scores: the fp64 sums are exact, so each mean is the rational mean."""
    rng = np.random.default_rng(61)
    r = rng.integers(-1000, 1000, size=64 * 20).astype(np.float64)
    m = S.block_scores(r, 3, 17)
    assert np.all(np.isneginf(m[:3])) and m.shape == (17,)
    for j in range(3, 17):
        want = Fraction(int(r[64 * j:64 * j + 64].sum()), 64)
        assert Fraction(m[j]) == want


def test_block_means_follow_sequential_order():
    """A block whose ascending-order fp64 sum differs from other orders: the oracle
    adds its tokens one at a time from the first."""
    r = np.zeros(64)
    r[0], r[1], r[2] = 1e16, 1.0, -1e16     # (1e16 + 1) - 1e16 = 0 in fp64; 1 + (1e16 - 1e16) = 1
    m = S.block_scores(r, 0, 1)
    assert m[0] == 0.0 and not np.signbit(m[0])
    r2 = np.full(64, -0.0)
    assert not np.signbit(S.block_scores(r2, 0, 1)[0])      # +0.0, never -0.0


def test_block_topk_brute_force_with_ties():
    rng = np.random.default_rng(62)
    for _ in range(20):
        nb = int(rng.integers(1, 40))
        r = rng.integers(0, 4, size=64 * nb).astype(np.float64)   # many tied block means
        n = 64 * nb + int(rng.integers(0, 64))
        n_sink, n_window = int(rng.integers(0, 100)), int(rng.integers(0, 100))
        lo, hi = S.block_range(n, n_sink, n_window)
        m = S.block_scores(np.concatenate([r, np.zeros(64)]), lo, hi)
        k = int(rng.integers(0, nb + 3))
        got = S.topk_indices(m, lo, hi, k, nb + 3)
        means = {j: Fraction(int(r[64 * j:64 * j + 64].sum()), 64) for j in range(lo, hi)}
        brute = sorted(sorted(means, key=lambda j: (-means[j], j))[:k])
        assert got[got >= 0].tolist() == brute
        assert np.all(got[len(brute):] == -1)


def test_block_tokens_hand_example():
    toks = S.block_tokens(400, 4, 64, [3, 1, -1, 5, 0])   # candidates [1, 5): 1 and 3 kept
    want = list(range(4)) + list(range(64, 128)) + list(range(192, 256)) + list(range(336, 400))
    assert toks.tolist() == want
    assert S.attended_tokens("blocks", 400, 4, 64, [3, 1, -1, 5, 0]).tolist() == want


def test_planted_block_is_selected_first():
    """A block whose every token scores highest is kept before any other."""
    rng = np.random.default_rng(63)
    r = rng.normal(size=64 * 50)
    r[64 * 37:64 * 38] = 10.0
    m = S.block_scores(r, 0, 50)
    assert S.topk_indices(m, 0, 50, 1, 1).tolist() == [37]


def test_all_blocks_kept_is_dense_attention():
    """Keeping every candidate block, with the window starting where the last
    candidate block ends, attends every token: the step equals dense attention
    over the same cache (1001 tokens after the append: blocks 0..13, window
    [896, 1001))."""
    w = W.sparse_blocks(n_ctx=1000, fmt="int4", top_blocks=100)
    w.n_sink, w.n_window = 0, 105
    res = ST.decode_step(w, append=True)
    wd = W.sparse_blocks(n_ctx=1000, fmt="int4", top_blocks=100)
    wd.mode, wd.score, wd.accumulate = "dense", None, False
    dense = ST.decode_step(wd, append=True)
    for (b, g), toks in res.tokens.items():
        assert toks.tolist() == list(range(1001))
    assert np.array_equal(res.o, dense.o) and np.array_equal(res.lse, dense.lse)


def test_step_ranks_blocks_by_mean_token_score():
    w = W.sparse_blocks(n_ctx=3000, fmt="fp16", top_blocks=5)
    res = ST.decode_step(w, append=False, pairs=[(0, 2)])
    hc = res.caches[(0, 2)]
    q = w.q[0, 8:12]
    ch = S.critical_channels(q, hc.kabs, 8)
    r = S.token_scores(q, hc.k16.astype(np.float64), ch)
    lo, hi = S.block_range(3000, 0, 0)
    assert (lo, hi) == (0, 46)
    m = res.scores[(0, 2)]
    for j in range(lo, hi):
        assert m[j] == sum(float(x) for x in r[64 * j:64 * j + 64]) / 64
    sel = res.sel[(0, 2)]
    order = sorted(range(lo, hi), key=lambda j: (-m[j], j))
    assert sel.tolist() == sorted(order[:5])
    toks = res.tokens[(0, 2)]
    assert toks.tolist() == sorted(t for j in sel for t in range(64 * j, 64 * j + 64))
    keys = hc.k16.astype(np.float64)
    vals = hc.v16.astype(np.float64)
    o, lse, _ = A.attend_group(q, keys[toks], vals[toks], w.sm_scale)
    assert np.array_equal(res.o[0, 8:12], o)
