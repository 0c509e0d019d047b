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

Readings taken (each listed in the design doc):
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
    (selected ids outside [n_sink, n - n_window) and -1 padding are ignored).
    """
    if mode in ("dense", "keep"):
        return np.arange(n)
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
