"""Pins for the oracle's attention, H2O update and whole-step composition (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attend as A
from oracle import quant as Q
from oracle import select as S
from oracle import step as ST

SM = float(np.float32(1.0 / np.sqrt(128)))


def _sdpa(q, k, v, scale):
    """torch's textbook attention in fp64 on the CPU: q [H, D], k/v [T, D]."""
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]       # [1, H, 1, D]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0].numpy()


def test_dense_fp16_equals_sdpa():
    rng = np.random.default_rng(41)
    q = rng.normal(size=(4, 128)).astype(np.float16)
    k = rng.normal(size=(777, 128)).astype(np.float16).astype(np.float64)
    v = rng.normal(size=(777, 128)).astype(np.float16).astype(np.float64)
    o, lse, logits = A.attend_group(q, k, v, SM)
    np.testing.assert_allclose(o, _sdpa(q, k, v, SM), rtol=1e-12, atol=1e-13)
    ref_lse = torch.logsumexp(torch.from_numpy(k @ q.astype(np.float64).T * SM), dim=0).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_lossless_codes_reduce_to_dense_attention():
    """All tokens kept and grid-exact codes: dequantized attention = fp16 dense attention."""
    rng = np.random.default_rng(42)
    n = 256
    ck = rng.integers(0, 16, size=(n, 128))
    ck[::64] = 0
    ck[1::64] = 15
    kf = (ck * 0.25 - 2.0)
    cv = rng.integers(0, 16, size=(n, 128))
    cv[:, 0] = 0
    cv[:, 1] = 15
    cv[:, 64] = 0
    cv[:, 65] = 15
    vf = cv * 0.125 - 1.0
    k16 = kf.astype(np.float16)
    v16 = vf.astype(np.float16)
    hc = ST.build_head_cache(k16, v16, "int4")
    keys, vals = ST.token_rows(hc)
    assert np.array_equal(keys, kf) and np.array_equal(vals, vf)
    q = rng.normal(size=(2, 128)).astype(np.float16)
    o, _, _ = A.attend_group(q, keys, vals, SM)
    np.testing.assert_allclose(o, _sdpa(q, kf, vf, SM), rtol=1e-12, atol=1e-13)


def test_single_token_and_uniform_logits():
    rng = np.random.default_rng(43)
    q = rng.normal(size=128).astype(np.float16)
    k = rng.normal(size=(1, 128))
    v = rng.normal(size=(1, 128))
    o, lse, lg = A.attend_head(q, k, v, SM)
    assert np.array_equal(o, v[0]) and lse == lg[0]
    kk = np.repeat(k, 50, axis=0)
    vv = rng.normal(size=(50, 128))
    o, lse, lg = A.attend_head(q, kk, vv, SM)
    np.testing.assert_allclose(o, vv.mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lg[0] + np.log(50), rtol=1e-14)
    o, lse, _ = A.attend_head(q, np.zeros((0, 128)), np.zeros((0, 128)), SM)
    assert np.all(o == 0) and lse == -np.inf


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(44)
    q = (rng.normal(size=(4, 128)) * 3).astype(np.float16)
    k = rng.normal(size=(1000, 128))
    v = rng.normal(size=(1000, 128))
    _, lse, logits = A.attend_group(q, k, v, SM)
    np.testing.assert_allclose(np.exp(logits - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)


def test_h2o_accumulation_is_column_sums():
    """After T steps, acc = column sums of the explicit attention matrices, over the group's heads."""
    rng = np.random.default_rng(45)
    n, G, T = 90, 4, 5
    k = rng.normal(size=(n, 128))
    v = rng.normal(size=(n, 128))
    acc = np.zeros(n)
    cols = torch.zeros(n, dtype=torch.float64)
    for step in range(T):
        q = rng.normal(size=(G, 128)).astype(np.float16)
        toks = np.sort(rng.choice(n, 60, replace=False))
        _, lse, logits = A.attend_group(q, k[toks], v[toks], SM)
        acc = A.h2o_update(acc, toks, logits, lse)
        attn = torch.softmax(torch.from_numpy(q.astype(np.float64)) @ torch.from_numpy(k[toks]).T * SM, dim=1)
        cols[torch.from_numpy(toks)] += attn.sum(dim=0)
        # each step adds exactly G of probability mass
        assert abs(acc.sum() - G * (step + 1)) < 1e-10
    np.testing.assert_allclose(acc, cols.numpy(), rtol=1e-12, atol=1e-14)


def test_gqa_group_equals_per_head_mha():
    rng = np.random.default_rng(46)
    q = rng.normal(size=(4, 128)).astype(np.float16)
    k = rng.normal(size=(64, 128))
    v = rng.normal(size=(64, 128))
    o, lse, _ = A.attend_group(q, k, v, SM)
    for h in range(4):
        oh, lh, _ = A.attend_head(q[h], k, v, SM)
        assert np.array_equal(o[h], oh) and lse[h] == lh


def test_step_tiers_and_attended_sets():
    """A small single-head workload: drop mode reads only sinks U top-k U window."""
    w = W.single_head_4k(n_ctx=300)
    res = ST.decode_step(w, append=True)
    hc = res.caches[(0, 0)]
    assert hc.n == 301 and hc.nq == 256
    sel = res.sel[(0, 0)]
    toks = res.tokens[(0, 0)]
    want = set(range(4)) | set(int(t) for t in sel if t >= 0) | set(range(301 - 64, 301))
    assert set(toks.tolist()) == want
    # top-k came from [4, n - 64) and by exact score on the dequantized keys
    keys, _ = ST.token_rows(hc)
    r = S.token_scores(w.q[0, :1], keys, range(128))
    assert np.array_equal(r, res.scores[(0, 0)])
    assert np.array_equal(sel, S.topk_indices(r, 4, 301 - 64, 128, 128))
    # the fp16 tail is fp16, the rest dequantized
    assert np.array_equal(keys[256:], hc.k16[256:].astype(np.float64))
    assert np.array_equal(keys[:256], Q.dequant_keys(hc.k_code, hc.k_scale, hc.k_zero))


def test_keep_mode_reads_keep_set_in_fp16():
    w = W.batched_joint(batch=2, lo=300, hi=400, n_window=64)
    res = ST.decode_step(w, append=False)
    for (b, g), hc in res.caches.items():
        n = hc.n
        sel = res.sel[(b, g)]
        assert (sel >= 0).sum() == min(int(w.top_k[b]), n - 64 - 4)
        mask = S.keep_set(n, 4, 64, sel)
        keys, vals = ST.token_rows(hc, mask)
        assert np.array_equal(keys[mask], hc.k16[mask].astype(np.float64))
        q = w.q[b, 4 * g:4 * g + 4]
        o, lse, _ = A.attend_group(q, keys, vals, w.sm_scale)
        assert np.array_equal(res.o[b, 4 * g:4 * g + 4], o)
