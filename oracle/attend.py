"""Decode attention over the attended tokens, and the H2O score update (oracle).

Test infrastructure only.

Sources:
  * TailorKV article, section 2.1: attention weights are softmax(Q K^T / sqrt(d_h)).
  * Meeting-LLM article, section 8.1 (FlashDecoding-Sparse sketch): one decode
    step computes S = Q K^T over the active blocks, a softmax (kept online
    there), and O = P V.  The online rescale is an implementation device; the
    oracle computes the plain softmax it equals.
  * On-device KV article, section 3.2: dequantization feeds Q K^T and P V
    directly (fused); the oracle dequantizes exactly in fp64 first.
  * StreamingLLM / H2O survey, section 3.2 (H2O): cumulative attention scores
    per token, accumulated over decode steps.

Readings:
  * GQA: query head h reads KV head floor(h / G), G = Hq / Hkv (pages silent;
    Llama convention).
  * The scale is 1/sqrt(128) passed as a float32 value; lse is the natural log.
  * The H2O update of a KV head adds, for every attended token, the attention
    probabilities of all G query heads that read it; unattended tokens add 0.
"""
from __future__ import annotations

import numpy as np


def attend_head(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, sm_scale: float):
    """One query head over T tokens, fp64.

    q: float16 [D]; keys, vals: float64 [T, D].  Returns (o [D], lse, logits [T]).
    With T == 0: o = 0, lse = -inf.
    """
    if keys.shape[0] == 0:
        return np.zeros(q.shape[0]), -np.inf, np.zeros(0)
    logits = (keys @ q.astype(np.float64)) * np.float64(sm_scale)
    m = logits.max()
    e = np.exp(logits - m)
    z = e.sum()
    o = (e @ vals) / z
    return o, m + np.log(z), logits


def attend_group(q_grp: np.ndarray, keys: np.ndarray, vals: np.ndarray, sm_scale: float):
    """All G query heads of one KV head.  Returns (o [G, D], lse [G], logits [G, T])."""
    outs, lses, logs = [], [], []
    for h in range(q_grp.shape[0]):
        o, lse, lg = attend_head(q_grp[h], keys, vals, sm_scale)
        outs.append(o)
        lses.append(lse)
        logs.append(lg)
    return np.stack(outs), np.array(lses), np.stack(logs) if logs else np.zeros((0, 0))


def h2o_update(acc: np.ndarray, tokens: np.ndarray, logits: np.ndarray,
               lse: np.ndarray) -> np.ndarray:
    """acc[t] += sum_h exp(logit_{h,t} - lse_h) for the attended tokens (fp64 copy)."""
    out = acc.astype(np.float64).copy()
    if tokens.size:
        p = np.exp(logits - lse[:, None])       # [G, T]
        np.add.at(out, tokens, p.sum(axis=0))
    return out
