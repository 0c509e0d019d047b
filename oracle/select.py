"""Importance scoring and Top-K token selection (oracle; test infrastructure only).

Sources:
  * TailorKV article, section 2.3: channel importance s_i = |q_i| * max|K_i|
    over the query and the cached keys; the top ``critical_channels`` (8, its
    section 5.1 configuration) are kept; approximate attention scores use only
    those channels (critical query x critical key transpose); the K highest
    scoring tokens are loaded (typical K = 128; ``sparse_ratio`` 0.03 in 5.1).
  * Meeting-LLM article, section 2.2: query-aware scores S_qry (full q . k) and
    Top-K on them.
  * StreamingLLM / H2O survey, section 3.1: keep the first 4-8 "sink" tokens
    and a recent window (e.g. 2048 tokens); section 3.2: H2O keeps tokens with
    high cumulative attention score.

Readings taken:
  * GQA: a KV head serves G query heads; the channel importance uses the max
    over the group of |q_{h,c}|, and a token's score is the max over the group
    of the per-head scores.  Max is order-free, so the result is exact.
  * The query used for channel importance is this step's q (the article
    predicts it from layer l-1, which needs model weights).
  * max|K_c| runs over every token cached for the (sequence, KV head), taken on
    the fp16 values seen at append time.
  * Scores are fp64 sums of exact fp16 x fp16 (or fp16 x dequantized) products,
    added one channel at a time in ascending channel order starting from +0.0,
    then +0.0 is added to turn -0.0 into +0.0.  No 1/sqrt(d) (rank-invariant).
  * Top-K orders by (score descending, token index ascending), takes
    min(K, #candidates), and returns indices ascending, padded with -1.
  * Sinks and the recent window are kept outside the Top-K: candidates are the
    tokens in [n_sink, n - n_window).

Block-granular selection (meeting-LLM article, part 2, section 1.1, and its
section 8.1: importance is averaged over 64- or 128-token blocks and the top
P% of blocks are kept, trading a little accuracy for contiguous reads).
Readings taken:
  * A block is a 64-token quantization group (the smaller of the two sizes,
    and the unit the codes are stored in); only complete blocks are
    candidates, and only those lying wholly inside [n_sink, n - n_window).
  * A block's importance is the mean of its tokens' ranking scores (the same
    per-token score as above): an fp64 sum over its tokens in ascending order
    from +0.0, divided by 64 (exact: a power of two), plus +0.0.
  * The kept blocks are the top k by (mean desc, block index asc), returned
    ascending and -1 padded, like the token Top-K; the attended set is the
    sinks, every token of the kept blocks, and the recent window.
"""
from __future__ import annotations

import numpy as np


def critical_channels(q_grp: np.ndarray, kabs: np.ndarray, n_crit: int) -> np.ndarray:
    """Top ``n_crit`` channels by max_h |q_{h,c}| * max_t |K_{t,c}|, ascending.

    q_grp: float16 [G, D]; kabs: float16 [D] (max |K| per channel).
    """
    d = q_grp.shape[1]
    qmax = np.abs(q_grp.astype(np.float64)).max(axis=0)
    s = qmax * kabs.astype(np.float64)
    order = sorted(range(d), key=lambda c: (-s[c], c))
    return np.array(sorted(order[: min(n_crit, d)]), dtype=np.int32)


def token_scores(q_grp: np.ndarray, keys: np.ndarray, channels) -> np.ndarray:
    """Ranking score per token: max over heads of sum_{c in channels} q_{h,c} k_{t,c}.

    q_grp: float16 [G, D]; keys: float64 [N, D] (fp16 values or exact dequantized
    values); channels: ascending channel ids.  Sequential fp64 sum per head.
    """
    qf = q_grp.astype(np.float64)
    n = keys.shape[0]
    best = None
    for h in range(qf.shape[0]):
        acc = np.zeros(n, dtype=np.float64)
        for c in channels:
            acc = acc + qf[h, c] * keys[:, c]
        best = acc if best is None else np.maximum(best, acc)
    return best + 0.0


def topk_indices(r: np.ndarray, lo: int, hi: int, k: int, k_max: int) -> np.ndarray:
    """The k best candidates in [lo, hi) by (r desc, t asc), ascending, -1 padded to k_max."""
    lo = max(lo, 0)
    hi = min(hi, r.shape[0])
    cand = np.arange(lo, hi) if hi > lo else np.zeros(0, np.int64)
    take = min(max(k, 0), cand.size, k_max)    # the output holds k_max entries
    # lexsort: last key is primary; -r descending, then t ascending
    order = np.lexsort((cand, -r[cand])) if cand.size else cand
    chosen = np.sort(cand[order[:take]])
    out = np.full(k_max, -1, dtype=np.int32)
    out[:take] = chosen
    return out


def attended_tokens(mode: str, n: int, n_sink: int, n_window: int, sel) -> np.ndarray:
    """Token ids attended in one step, ascending.

    dense / keep: every cached token; drop: sinks U selected U recent window
    (selected ids outside [n_sink, n - n_window) and -1 padding are ignored);
    blocks: sel holds block ids (see block_tokens).
    """
    if mode in ("dense", "keep"):
        return np.arange(n)
    if mode == "blocks":
        return block_tokens(n, n_sink, n_window, sel)
    sinks = np.arange(min(n_sink, n))
    w0 = max(n - n_window, 0)
    window = np.arange(max(w0, min(n_sink, n)), n)
    s = np.asarray(sel)
    s = s[(s >= n_sink) & (s < w0)]
    return np.unique(np.concatenate([sinks, s.astype(np.int64), window]))


def keep_set(n: int, n_sink: int, n_window: int, sel) -> np.ndarray:
    """Boolean [n]: sinks U selected U window (the fp16 tier in keep mode)."""
    m = np.zeros(n, dtype=bool)
    m[attended_tokens("drop", n, n_sink, n_window, sel)] = True
    return m


BLOCK = 64


def block_range(n: int, n_sink: int, n_window: int):
    """Candidate blocks [lo, hi): complete 64-token blocks inside [n_sink, n - n_window)."""
    lo = -(-max(n_sink, 0) // BLOCK)
    hi = max(n - n_window, 0) // BLOCK
    return lo, max(hi, lo)


def block_scores(r: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Mean token score of each candidate block, indexed by block id ([0, hi); -inf below lo).

    Each block's tokens are added one at a time in ascending order from +0.0
    (vectorized over blocks only), then divided by 64.
    """
    out = np.full(max(hi, 0), -np.inf)
    if hi <= lo:
        return out
    blocks = np.arange(lo, hi)
    acc = np.zeros(blocks.size, dtype=np.float64)
    for i in range(BLOCK):
        acc = acc + r[BLOCK * blocks + i]
    out[lo:hi] = acc / BLOCK + 0.0
    return out


def block_tokens(n: int, n_sink: int, n_window: int, blocks) -> np.ndarray:
    """Sinks, every token of the kept candidate blocks, and the recent window, ascending."""
    lo, hi = block_range(n, n_sink, n_window)
    b = np.asarray(blocks, dtype=np.int64)
    b = b[(b >= lo) & (b < hi)]
    toks = (BLOCK * b[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
    sinks = np.arange(min(n_sink, n))
    window = np.arange(max(max(n - n_window, 0), min(n_sink, n)), n)
    return np.unique(np.concatenate([sinks, toks, window]).astype(np.int64))


def topk_mass(probs: np.ndarray, k: int) -> float:
    """Sum of the k largest attention probabilities of one query row (fp64).

    TailorKV article, section 2.1 (dense preference score): for each of the last
    n_q queries, the top-k entries of its softmax row are taken and their
    probabilities summed.  The sum does not depend on which of several equal
    entries count as the k-th.
    """
    p = np.sort(np.asarray(probs, dtype=np.float64))[::-1]
    return float(p[: max(0, min(int(k), p.size))].sum())


def dense_preference(masses) -> float:
    """P = n_q - sum over the n_q queries of their top-k probability mass."""
    m = np.asarray(masses, dtype=np.float64)
    return float(m.size - m.sum())


def quantization_friendly(P: float, tau: float = 0.2) -> bool:
    """A layer whose attention spreads beyond its top-k entries (P above tau) is
    quantization-friendly; one that concentrates in them is sparsity-friendly.
    (The comparison sign is lost in the page's text; this reading matches its
    example, where the dense layer 0 scores 0.7178 and layer 16 0.0473.)"""
    return bool(P > tau)
