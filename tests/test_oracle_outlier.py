"""Pins for the oracle's outlier channels (meeting-LLM article, section 8.2:
channels chosen by variance offline, their K and V kept at full precision beside
the INT4 main store).  CPU only."""
from fractions import Fraction

import numpy as np
import torch

import workloads as W
from oracle import attend as A
from oracle import quant as Q
from oracle import step as ST

SM = float(np.float32(1.0 / np.sqrt(128)))


def _exact_variance(col):
    """Population variance of one column in exact rational arithmetic."""
    xs = [Fraction(float(x)) for x in col]
    mean = sum(xs) / len(xs)
    return sum((x - mean) ** 2 for x in xs) / len(xs)


def test_variance_ranking_brute_force():
    """Tiny matrices with planted ties: the choice equals an exact-rational ranking
    under (variance desc, channel asc)."""
    rng = np.random.default_rng(71)
    for trial in range(20):
        n, d = int(rng.integers(2, 9)), int(rng.integers(2, 12))
        x = rng.integers(-4, 5, size=(n, d)).astype(np.float16) * np.float16(0.5)
        if d > 3:
            x[:, 2] = x[:, 1]            # equal variance: the lower channel wins
            x[:, 3] = x[:, 1] + np.float16(1)   # a shift keeps the variance
        for m in range(0, d + 1):
            var = [_exact_variance(x[:, c]) for c in range(d)]
            want = sorted(sorted(range(d), key=lambda c: (-var[c], c))[:m])
            assert Q.outlier_channels(x, m).tolist() == want, (trial, m)


def test_variance_finds_planted_channels():
    """The synthetic layers scale 3 channels per KV head by 8 (64x the variance):
    the variance analysis of the first 4096 tokens names exactly those."""
    w = W.int4_dense(4096)
    for g in range(w.hkv):
        got = Q.outlier_channels(w.k[0, :4096, g], 3)
        assert got.tolist() == w.planted[g].tolist()


def test_outlier_channels_kept_exactly_and_others_unchanged():
    rng = np.random.default_rng(72)
    k16 = rng.normal(size=(200, 128)).astype(np.float32)
    ch = np.array([5, 77, 126])
    k16[:, ch] *= 8
    k16 = k16.astype(np.float16)
    code0, s0, z0 = Q.quantize_keys(k16, 4)
    code, s, z, k_out = Q.quantize_keys_outliers(k16, 4, ch)
    assert code.shape == (192, 128) and k_out.shape == (192, 3) and k_out.dtype == np.float16
    # the main store holds nothing on the outlier channels
    assert not code[:, ch].any() and not s[:, ch].astype(np.float32).any()
    assert not np.signbit(s[:, ch]).any() and not z[:, ch].astype(np.float32).any()
    other = np.setdiff1d(np.arange(128), ch)
    # per-channel groups are independent: the other channels are quantized as before
    assert np.array_equal(code[:, other], code0[:, other])
    assert np.array_equal(s[:, other].view(np.uint16), s0[:, other].view(np.uint16))
    assert np.array_equal(z[:, other].view(np.uint16), z0[:, other].view(np.uint16))
    kd = Q.dequant_keys_outliers(code, s, z, ch, k_out)
    assert np.array_equal(kd[:, ch], k16[:192, ch].astype(np.float64))
    assert np.array_equal(kd[:, other], Q.dequant_keys(code0, s0, z0)[:, other])


def test_value_outliers_leave_the_main_store_alone():
    """V groups run per token across channels: whatever the outlier channels hold
    (here huge values, then copies of a neighbour), every other channel's codes and
    every group's scale and zero are the same, the outlier codes are 0, and the
    dequantized outlier channels are the fp16 values."""
    rng = np.random.default_rng(74)
    v = rng.normal(size=(192, 128)).astype(np.float16)
    ch = np.array([7, 64, 90])
    big = v.copy()
    big[:, ch] = (rng.normal(size=(192, 3)) * 3000).astype(np.float16)
    tame = v.copy()
    tame[:, ch] = v[:, ch + 1]          # values inside the other channels' range
    c1, s1, z1, vo1 = Q.quantize_values_outliers(big, 4, ch)
    c2, s2, z2, vo2 = Q.quantize_values_outliers(tame, 4, ch)
    other = np.setdiff1d(np.arange(128), ch)
    assert np.array_equal(c1[:, other], c2[:, other])
    assert np.array_equal(s1.view(np.uint16), s2.view(np.uint16))
    assert np.array_equal(z1.view(np.uint16), z2.view(np.uint16))
    assert not c1[:, ch].any() and not c2[:, ch].any()
    # with tame outliers the groups equal plain quantization's (the range is the same)
    c0, s0, z0 = Q.quantize_values(tame, 4)
    assert np.array_equal(c2[:, other], c0[:, other])
    assert np.array_equal(s2.view(np.uint16), s0.view(np.uint16))
    vd = Q.dequant_values_outliers(c1, s1, z1, ch, vo1)
    assert np.array_equal(vd[:, ch], big[:, ch].astype(np.float64))
    assert np.array_equal(vd[:, other], Q.dequant_values(c2, s2, z2)[:, other])


def test_value_isolation_reduces_output_error():
    """Planted V outlier channels (x20) blow up their token groups' scales; isolating
    them brings the attention output closer to fp16 attention."""
    rng = np.random.default_rng(75)
    k = rng.normal(size=(1024, 128)).astype(np.float16)
    v = rng.normal(size=(1024, 128)).astype(np.float32)
    ch = np.array([11, 70])
    v[:, ch] *= 20
    v = v.astype(np.float16)
    q = rng.normal(size=(4, 128)).astype(np.float16)
    ref, _, _ = A.attend_group(q, k.astype(np.float64), v.astype(np.float64), SM)
    err = {}
    for name, oc, ov in (("plain", None, True), ("k_only", ch, False), ("k_and_v", ch, True)):
        keys, vals = ST.token_rows(ST.build_head_cache(k, v, "int4", oc, ov))
        o, _, _ = A.attend_group(q, keys, vals, SM)
        err[name] = np.abs(o - ref).mean()
    assert err["k_and_v"] < 0.5 * err["k_only"], err


def test_outliers_with_lossless_main_reduce_to_dense_attention():
    """Main channels on an exact INT4 grid, outlier channels arbitrary fp16: the
    dequantized keys are the fp16 keys, so attention is textbook fp16 attention."""
    rng = np.random.default_rng(73)
    n = 192
    ck = rng.integers(0, 16, size=(n, 128))
    ck[::64] = 0
    ck[1::64] = 15
    kf = ck * 0.25 - 2.0
    ch = np.array([3, 64, 100])
    kf[:, ch] = rng.normal(size=(n, 3)).astype(np.float16).astype(np.float64) * 37.0
    k16 = kf.astype(np.float16)
    kf = k16.astype(np.float64)
    cv = rng.integers(0, 16, size=(n, 128))
    cv[:, 0] = 0
    cv[:, 1] = 15
    cv[:, 65] = 0
    cv[:, 66] = 15
    vf = cv * 0.125 - 1.0
    vf[:, ch] = rng.normal(size=(n, 3)).astype(np.float16).astype(np.float64) * 50.0
    v16 = vf.astype(np.float16)
    hc = ST.build_head_cache(k16, v16, "int4", ch)
    keys, vals = ST.token_rows(hc)
    assert np.array_equal(keys, kf)
    assert np.array_equal(vals, v16.astype(np.float64))
    hc_plain = ST.build_head_cache(k16, v16, "int4")
    assert not np.array_equal(ST.token_rows(hc_plain)[0], kf)   # without the store: lossy
    assert not np.array_equal(ST.token_rows(hc_plain)[1], v16.astype(np.float64))
    q = rng.normal(size=(4, 128)).astype(np.float16)
    vv = v16.astype(np.float64)
    o, _, _ = A.attend_group(q, keys, vals, SM)
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    kt = torch.from_numpy(kf)[None, None].expand(1, 4, -1, -1)
    vt = torch.from_numpy(vv)[None, None].expand(1, 4, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM)[0, :, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_isolation_reduces_logit_error_on_the_planted_layer():
    """The accuracy effect the section is about: with the planted channels in
    fp16 the logits of the quantized keys move closer to the fp16 logits."""
    w = W.int4_outlier_dense(2048)
    g = 0
    k16, v16 = w.k[0, :2048, g], w.v[0, :2048, g]
    q = w.q[0, :4].astype(np.float64)
    exact = k16.astype(np.float64) @ q.T
    err = {}
    for name, oc in (("plain", None), ("outlier", w.outlier_ch[g])):
        keys, _ = ST.token_rows(ST.build_head_cache(k16, v16, "int4", oc))
        err[name] = np.abs(keys @ q.T - exact).mean()
    assert err["outlier"] < 0.8 * err["plain"], err


def test_step_uses_the_outlier_store():
    """decode_step with the workload's outlier list equals attention over the
    keys rebuilt by hand from the outlier store."""
    w = W.int4_outlier_dense(640)
    res = ST.decode_step(w, append=False, pairs=[(0, 1)])
    hc = res.caches[(0, 1)]
    assert hc.out_ch.tolist() == w.outlier_ch[1].tolist()
    keys = Q.dequant_keys(hc.k_code, hc.k_scale, hc.k_zero)
    keys[:, hc.out_ch] = w.k[0, :640, 1][:, hc.out_ch].astype(np.float64)
    vals = Q.dequant_values(hc.v_code, hc.v_scale, hc.v_zero)
    vals[:, hc.out_ch] = w.v[0, :640, 1][:, hc.out_ch].astype(np.float64)
    o, lse, _ = A.attend_group(w.q[0, 4:8], keys, vals, w.sm_scale)
    np.testing.assert_allclose(res.o[0, 4:8], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.lse[0, 4:8], lse, rtol=1e-13)
