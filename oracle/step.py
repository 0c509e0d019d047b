"""One decode step of the jointly compressed KV cache, end to end (oracle).

Test infrastructure only.  Composes ``quant``, ``select`` and ``attend`` in the
order a decode step runs: append the step's token (quantizing every 64-token
group it completes), pick critical channels and score tokens, select Top-K,
attend over the attended set with each token read from its tier, and add this
step's probabilities to the cumulative scores.

Tiers per token (meeting-LLM article, section 3.1: hot tokens at full
precision, warm tokens quantized; TailorKV article, section 3.1: a quantized
buffer beside an fp16 buffer of the key tokens):
  * fp16 format: every token is fp16.
  * int4 / int1, dense or drop mode: tokens of complete 64-token groups are
    dequantized codes, the incomplete last group is fp16.
  * fp8: every token is its E4M3 codes, decoded (encoded when appended).
  * keep mode: sinks, selected tokens and the recent window are fp16; the rest
    as in dense mode.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

from . import attend as A
from . import quant as Q
from . import select as S

BITS = {"int4": 4, "int1": 1}


@dataclasses.dataclass
class HeadCache:
    """What the cache holds for one (sequence, KV head) after appending."""
    n: int
    nq: int
    k16: np.ndarray             # [n, D] fp16 (all tokens, as appended)
    v16: np.ndarray
    kabs: np.ndarray            # [D] fp16 max |K| over the n tokens
    k_code: Optional[np.ndarray] = None   # [nq, D] uint8
    k_scale: Optional[np.ndarray] = None  # [nq/64, D] f16
    k_zero: Optional[np.ndarray] = None
    v_code: Optional[np.ndarray] = None   # [nq, D] uint8
    v_scale: Optional[np.ndarray] = None  # [nq, D/64] f16
    v_zero: Optional[np.ndarray] = None
    out_ch: Optional[np.ndarray] = None   # [m] K outlier channels (int4), ascending
    k_out: Optional[np.ndarray] = None    # [nq, m] f16 their K values
    v_out: Optional[np.ndarray] = None    # [nq, m] f16 their V values (V isolated too)


def build_head_cache(k16: np.ndarray, v16: np.ndarray, fmt: str,
                     out_ch: Optional[np.ndarray] = None, outlier_v: bool = True) -> HeadCache:
    """Cache contents after appending the fp16 rows k16, v16 [n, D].

    out_ch: channels kept at fp16 beside the INT4 codes (outlier channels), for
    K, and for V too when outlier_v.
    """
    n = k16.shape[0]
    kabs = np.abs(k16).max(axis=0) if n else np.zeros(k16.shape[1], np.float16)
    hc = HeadCache(n=n, nq=n, k16=k16, v16=v16, kabs=kabs.astype(np.float16))
    if fmt == "fp8":
        hc.k_code, hc.v_code = Q.encode_fp8(k16), Q.encode_fp8(v16)
    elif fmt in BITS:
        b = BITS[fmt]
        if out_ch is not None and len(out_ch):
            assert fmt == "int4"
            hc.out_ch = np.asarray(out_ch, dtype=np.int32)
            hc.k_code, hc.k_scale, hc.k_zero, hc.k_out = Q.quantize_keys_outliers(k16, b, hc.out_ch)
        else:
            hc.k_code, hc.k_scale, hc.k_zero = Q.quantize_keys(k16, b)
        if hc.out_ch is not None and outlier_v:
            hc.v_code, hc.v_scale, hc.v_zero, hc.v_out = Q.quantize_values_outliers(v16, b, hc.out_ch)
        else:
            hc.v_code, hc.v_scale, hc.v_zero = Q.quantize_values(v16, b)
        hc.nq = hc.k_code.shape[0]
    return hc


def token_rows(hc: HeadCache, fp16_mask: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 K~, V~ [n, D]: dequantized for quantized tokens, fp16 values otherwise."""
    keys = hc.k16.astype(np.float64)
    vals = hc.v16.astype(np.float64)
    if hc.k_code is not None and hc.k_scale is None:   # fp8: every row from its codes
        keys = Q.decode_fp8(hc.k_code)
        vals = Q.decode_fp8(hc.v_code)
    elif hc.k_code is not None and hc.nq:
        if hc.out_ch is not None:
            kq = Q.dequant_keys_outliers(hc.k_code, hc.k_scale, hc.k_zero, hc.out_ch, hc.k_out)
        else:
            kq = Q.dequant_keys(hc.k_code, hc.k_scale, hc.k_zero)
        if hc.v_out is not None:
            vq = Q.dequant_values_outliers(hc.v_code, hc.v_scale, hc.v_zero, hc.out_ch, hc.v_out)
        else:
            vq = Q.dequant_values(hc.v_code, hc.v_scale, hc.v_zero)
        quant = np.ones(hc.nq, dtype=bool)
        if fp16_mask is not None:
            quant &= ~fp16_mask[: hc.nq]
        keys[: hc.nq][quant] = kq[quant]
        vals[: hc.nq][quant] = vq[quant]
    return keys, vals


@dataclasses.dataclass
class StepResult:
    caches: Dict[Tuple[int, int], HeadCache]
    channels: Dict[Tuple[int, int], np.ndarray]
    scores: Dict[Tuple[int, int], np.ndarray]
    sel: Dict[Tuple[int, int], np.ndarray]
    tokens: Dict[Tuple[int, int], np.ndarray]          # attended token ids
    logits: Dict[Tuple[int, int], np.ndarray]          # [G, T] natural-log units
    o: np.ndarray                                      # [B, Hq, D] fp64
    lse: np.ndarray                                    # [B, Hq]
    acc: Optional[np.ndarray]                          # [B, Hkv, cap] fp64 after update


def decode_step(w, append: bool = True, pairs=None, k_max: Optional[int] = None) -> StepResult:
    """Run one decode step of workload ``w`` (a ``workloads.Workload``).

    append: add w.k_new / w.v_new to the cache first (a full step); otherwise
    attend over exactly the cached n_b tokens.  pairs: optional list of
    (b, g) to compute (a bounded sample); the rest of o/lse stay NaN.
    """
    B, G, D = w.batch, w.group, w.k.shape[-1]
    o = np.full((B, w.hq, D), np.nan)
    lse = np.full((B, w.hq), np.nan)
    acc = None if w.acc is None else w.acc.astype(np.float64).copy()
    res = StepResult({}, {}, {}, {}, {}, {}, o, lse, acc)
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(w.hkv)]
    for b, g in pairs:
        n0 = int(w.seq_lens[b])
        k16 = w.k[b, :n0, g]
        v16 = w.v[b, :n0, g]
        if append:
            k16 = np.concatenate([k16, w.k_new[b, :, g]])
            v16 = np.concatenate([v16, w.v_new[b, :, g]])
        n = k16.shape[0]
        oc = None if getattr(w, "outlier_ch", None) is None else w.outlier_ch[g]
        hc = build_head_cache(k16, v16, w.fmt, oc, getattr(w, "outlier_v", True))
        res.caches[(b, g)] = hc
        q_grp = w.q[b, g * G:(g + 1) * G]

        sel = np.zeros(0, np.int32)
        if w.score is not None:
            kk = int(w.top_k[b])
            km = kk if k_max is None else k_max
            lo, hi = w.n_sink, n - w.n_window
            if w.score == "external":
                r = w.acc[b, g, :n].astype(np.float64) + 0.0
            else:
                if w.score == "critical":
                    ch = S.critical_channels(q_grp, hc.kabs, w.n_crit)
                else:
                    ch = np.arange(D, dtype=np.int32)
                res.channels[(b, g)] = ch
                keys, _ = token_rows(hc)
                r = S.token_scores(q_grp, keys, ch)
            if w.granule == "block":   # rank 64-token blocks by their mean score
                lo, hi = S.block_range(n, w.n_sink, w.n_window)
                r = S.block_scores(r, lo, hi)
            res.scores[(b, g)] = r
            sel = S.topk_indices(r, lo, hi, kk, km)
            res.sel[(b, g)] = sel

        mask = S.keep_set(n, w.n_sink, w.n_window, sel) if w.mode == "keep" else None
        keys, vals = token_rows(hc, mask)
        toks = S.attended_tokens(w.mode, n, w.n_sink, w.n_window, sel)
        og, lg, logits = A.attend_group(q_grp, keys[toks], vals[toks], w.sm_scale)
        o[b, g * G:(g + 1) * G] = og
        lse[b, g * G:(g + 1) * G] = lg
        res.tokens[(b, g)] = toks
        res.logits[(b, g)] = logits
        if w.accumulate and acc is not None:
            acc[b, g] = A.h2o_update(acc[b, g], toks, logits, lg)
    return res
