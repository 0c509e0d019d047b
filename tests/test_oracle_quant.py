"""Pins for the oracle's quantizer against the pages and closed forms (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_worked.json")


def _group(head, fill):
    x = np.full(64, fill, dtype=np.float16)
    x[: len(head)] = np.array(head, dtype=np.float16)
    return x


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked_examples(case):
    """Hand-derived applications of the printed quantizer (TailorKV section 2.2)."""
    x = _group(case["head"], case["fill"])
    code, s, z = Q.quantize_groups(x[None], case["bits"])
    assert float(s[0]) == case["scale"]
    assert float(z[0]) == case["zero"]
    if case.get("zero_sign_positive"):
        assert not np.signbit(z[0])
    h = len(case["head"])
    assert code[0, :h].tolist() == case["codes_head"]
    assert np.all(code[0, h:] == case["code_fill"])


def _random_groups(rng, n, scale_exp_lo=-6, scale_exp_hi=6):
    mag = 2.0 ** rng.uniform(scale_exp_lo, scale_exp_hi, size=(n, 1))
    off = rng.normal(size=(n, 1)) * mag * 3
    return (rng.normal(size=(n, 64)) * mag + off).astype(np.float16)


@pytest.mark.parametrize("bits", [4, 1])
def test_error_bound_closed_form(bits):
    """|x - dequant(x)| <= s * (1/2 + 2^-18) whenever the fp16 scale is normal.

    Derivation: x >= min = z, so (x - z)/s >= 0 and the code is never clamped
    below; (max - min)/s16 <= (2^b - 1)(1 + 2^-11)(1 + 2^-23) < 2^b - 1/2, so it
    is never clamped above; rounding to the nearest integer costs <= s/2 and the
    two fp32 roundings (sub, div) cost <= 2 * 2^-24 * 15.01 s < 2^-18 s.
    """
    rng = np.random.default_rng(11)
    x = _random_groups(rng, 20000)
    code, s, z = Q.quantize_groups(x, bits)
    xh = Q.dequantize(code, s[:, None], z[:, None])
    err = np.abs(x.astype(np.float64) - xh)
    sf = s.astype(np.float64)[:, None]
    normal = s.astype(np.float64) >= 2.0 ** -14
    bound = sf * (0.5 + 2.0 ** -18)
    assert normal.mean() > 0.9
    assert np.all(err[normal] <= bound[normal])
    assert code.max() <= 2 ** bits - 1


@pytest.mark.parametrize("bits", [4, 1])
def test_min_and_max_map_to_end_codes(bits):
    rng = np.random.default_rng(12)
    x = _random_groups(rng, 5000)
    code, s, z = Q.quantize_groups(x, bits)
    xf = x.astype(np.float32)
    nz = s != 0
    amin = xf.argmin(axis=1)
    amax = xf.argmax(axis=1)
    r = np.arange(x.shape[0])
    assert np.all(code[r, amin] == 0)
    assert np.all(code[r[nz], amax[nz]] == 2 ** bits - 1)
    # zero point is the group minimum (as fp16, +0.0 for -0.0)
    assert np.array_equal(z.astype(np.float32), xf.min(axis=1) + 0.0)


@pytest.mark.parametrize("bits", [4, 1])
def test_lossless_grid_roundtrip(bits):
    """Values z + c*s with s = 2^-k and z a multiple of s give back c, s, z exactly."""
    rng = np.random.default_rng(13)
    top = 2 ** bits - 1
    for k in range(0, 8):
        s = 2.0 ** -k
        c = rng.integers(0, top + 1, size=(200, 64))
        c[:, 0] = 0
        c[:, 1] = top
        z = rng.integers(-40, 40, size=(200, 1)) * s
        x = (z + c * s).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), z + c * s)  # exactly representable
        code, s16, z16 = Q.quantize_groups(x, bits)
        assert np.array_equal(code, c)
        assert np.all(s16.astype(np.float64) == s)
        assert np.array_equal(z16.astype(np.float64), z[:, 0] + 0.0)
        # idempotence: quantizing the dequantized values changes nothing
        xh = Q.dequantize(code, s16[:, None], z16[:, None]).astype(np.float16)
        code2, _, _ = Q.quantize_groups(xh, bits)
        assert np.array_equal(code2, code)


def test_one_bit_is_a_midpoint_threshold():
    """1-bit: code = [x - min > s/2], away from one-ulp neighbourhoods of the midpoint."""
    rng = np.random.default_rng(14)
    x = _random_groups(rng, 5000)
    code, s, z = Q.quantize_groups(x, 1)
    d = x.astype(np.float64) - z.astype(np.float64)[:, None]
    half = s.astype(np.float64)[:, None] / 2
    far = np.abs(d - half) > 1e-3 * np.maximum(half, 1e-30)
    expect = (d > half).astype(np.uint8)
    assert np.array_equal(code[far], expect[far])


def test_key_groups_run_over_tokens_per_channel():
    """K: one (scale, zero) per channel per 64 tokens (TailorKV 2.2 'per channel').

    K[t, c] = (t % 16) * 2^-(c % 4) + (c % 8), exact in fp16: each channel's
    group spans codes 0..15 with scale 2^-(c%4) and zero c%8; a transposed
    grouping would mix channels.
    """
    t = np.arange(128)[:, None]
    c = np.arange(128)[None, :]
    kf = (t % 16) * 2.0 ** -(c % 4) + (c % 8)
    k = kf.astype(np.float16)
    assert np.array_equal(k.astype(np.float64), kf)
    code, s, z = Q.quantize_keys(k, 4)
    assert code.shape == (128, 128) and s.shape == (2, 128)
    assert np.array_equal(s.astype(np.float64), np.broadcast_to(2.0 ** -(np.arange(128) % 4), (2, 128)))
    assert np.array_equal(z.astype(np.float64), np.broadcast_to(np.arange(128.0) % 8, (2, 128)))
    assert np.array_equal(code, np.broadcast_to(t % 16, (128, 128)))


def test_value_groups_run_over_channels_per_token():
    """V: one (scale, zero) per token per 64 channels.

    V[t, c] = (c % 16) * 2^-(t % 3) + (t % 8) + 32*(c // 64), exact in fp16.
    """
    t = np.arange(64)[:, None]
    c = np.arange(128)[None, :]
    vf = (c % 16) * 2.0 ** -(t % 3) + (t % 8) + 32 * (c // 64)
    v = vf.astype(np.float16)
    assert np.array_equal(v.astype(np.float64), vf)
    code, s, z = Q.quantize_values(v, 4)
    assert s.shape == (64, 2)
    assert np.array_equal(s.astype(np.float64), np.repeat(2.0 ** -(np.arange(64) % 3)[:, None], 2, axis=1))
    assert np.array_equal(z.astype(np.float64), (np.arange(64) % 8)[:, None] + np.array([[0.0, 32.0]]))
    assert np.array_equal(code, np.broadcast_to(c % 16, (64, 128)))


def test_incomplete_group_stays_out():
    rng = np.random.default_rng(15)
    k = rng.normal(size=(100, 128)).astype(np.float16)
    code, s, z = Q.quantize_keys(k, 4)
    assert code.shape == (64, 128) and s.shape == (1, 128)
    vc, vs, vz = Q.quantize_values(k, 1)
    assert vc.shape == (64, 128) and vs.shape == (64, 2)


def test_dequant_keys_expands_group_parameters():
    code = np.tile((np.arange(64) % 16)[:, None], (1, 128)).astype(np.uint8)
    s = np.full((1, 128), 0.5, np.float16)
    z = np.full((1, 128), -2.0, np.float16)
    kq = Q.dequant_keys(code, s, z)
    assert np.array_equal(kq, (np.arange(64) % 16)[:, None] * 0.5 - 2.0 + np.zeros((1, 128)))


def test_signed_zero_groups_store_positive_zeros():
    x = np.zeros(64, np.float16)
    x[::2] = -0.0
    for bits in (4, 1):
        code, s, z = Q.quantize_groups(x[None], bits)
        assert s[0] == 0 and not np.signbit(s[0]) and not np.signbit(z[0])
        assert np.all(code == 0)


def test_one_bit_scale_saturates_at_the_largest_fp16():
    """A 1-bit group whose range exceeds 65504 stores scale 65504 (not infinity): the
    codes stay a midpoint threshold against it and every dequantized value is finite.
    Hand values: z = -40000; (x - z) / 65504 is 0, 1.22, exactly 0.5 (-> 0, half to
    even), 0.50049 and 0.61 for x = -40000, 40000, -7248, -7216, 0."""
    x = _group([-40000.0, 40000.0, -7248.0, -7216.0, 0.0], 0.0)
    code, s, z = Q.quantize_groups(x[None], 1)
    assert s[0] == np.float16(65504.0) and np.isfinite(s[0])
    assert float(z[0]) == -40000.0
    assert code[0, :5].tolist() == [0, 1, 0, 1, 1]
    assert np.all(np.isfinite(Q.dequantize(code, s[:, None], z[:, None])))
    # INT4 cannot reach it: the widest fp16 range over 15 levels is below 65504
    code4, s4, _ = Q.quantize_groups(_group([-65504.0, 65504.0], 0.0)[None], 4)
    assert float(s4[0]) == float(np.float16(np.float32(131008.0) / np.float32(15.0)))
