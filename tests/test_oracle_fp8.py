"""Pins for the oracle's FP8 (E4M3) warm tier (meeting-LLM article section 6.2; KV
compression survey section 2).  CPU only."""
from fractions import Fraction

import numpy as np

import workloads as W
from oracle import attend as A
from oracle import quant as Q
from oracle import step as ST

SM = float(np.float32(1.0 / np.sqrt(128)))


def _all_finite_fp16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    return x[np.isfinite(x)]


def test_grid_closed_form():
    """The E4M3 magnitudes: 0, subnormals k 2^-9, then 8 per binade up to 448."""
    g = Q.FP8_MAG
    assert g[0] == 0 and g[1] == 2.0 ** -9 and g[7] == 7 * 2.0 ** -9
    assert g[8] == 2.0 ** -6 and g[0x38] == 1.0 and g[0x7E] == 448.0
    assert np.all(np.diff(g) > 0)
    for e in range(1, 16):
        for m in range(8):
            assert g[8 * e + m] == (1 + m / 8) * 2.0 ** (e - 7) if 8 * e + m < 0x7F else True


def test_hand_examples():
    x = np.array([1.0, -2.0, 448, 1000, -1000, 2 ** -9, 2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875,
                  0.0, -0.0, 15 * 2 ** -10, 464, 463.9, 0.3], np.float16)
    want = [0x38, 0xC0, 0x7E, 0x7E, 0xFE, 0x01, 0x00, 0x02, 0x38, 0x3A, 0x00, 0x80, 0x08, 0x7E,
            0x7E, 0x2A]
    assert Q.encode_fp8(x).tolist() == want
    # 0.3 (fp16 0.2998...) lies between 0.28125 (0x29) and 0.3125 (0x2A): nearer 0x2A


def test_every_fp16_against_exact_nearest_even():
    """All 63488 finite fp16 values: the code is the nearest grid value in exact
    rational arithmetic, ties to the even code, saturating past 448."""
    import bisect
    x = _all_finite_fp16()
    code = Q.encode_fp8(x)
    grid = [Fraction(v) for v in Q.FP8_MAG]
    for i, xv in enumerate(x):
        a = abs(Fraction(float(xv)))
        if a > grid[-1]:
            best = 0x7E
        else:
            j = bisect.bisect_left(grid, a)
            near = [c for c in (j - 1, j) if 0 <= c < len(grid)]
            dmin = min(abs(a - grid[c]) for c in near)
            best = min((c for c in near if abs(a - grid[c]) == dmin), key=lambda c: (c & 1, c))
        want = best | (0x80 if np.signbit(xv) else 0)
        assert code[i] == want, (float(xv), hex(code[i]), hex(want))


def test_error_bound_and_round_trip():
    """|x - x~| <= half an E4M3 ulp in range; grid values round-trip exactly."""
    x = _all_finite_fp16()
    xf = x.astype(np.float64)
    dec = Q.decode_fp8(Q.encode_fp8(x))
    inr = np.abs(xf) <= 448
    e = np.floor(np.log2(np.maximum(np.abs(xf[inr]), 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    assert np.all(np.abs(xf[inr] - dec[inr]) <= ulp / 2)
    assert np.all(dec[~inr] == np.sign(xf[~inr]) * 448)
    g = np.concatenate([Q.FP8_MAG, -Q.FP8_MAG]).astype(np.float16)
    assert np.array_equal(Q.decode_fp8(Q.encode_fp8(g)), g.astype(np.float64))


def test_fp8_step_attends_decoded_rows():
    """Dense decode over an fp8 cache is softmax attention over the decoded rows,
    every token included (no fp16 tail)."""
    w = W.fp8_dense(n_ctx=300)
    res = ST.decode_step(w, append=True, pairs=[(0, 1)])
    hc = res.caches[(0, 1)]
    keys, vals = ST.token_rows(hc)
    assert keys.shape[0] == 301
    assert np.array_equal(keys, Q.decode_fp8(Q.encode_fp8(hc.k16)))
    q = w.q[0, 4:8]
    o, lse, _ = A.attend_group(q, keys, vals, SM)
    assert np.array_equal(res.o[0, 4:8], o)
