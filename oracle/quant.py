"""Asymmetric min-max KV quantization (oracle; test infrastructure only).

Source: TailorKV article ("TailorKV's hybrid compression architecture"),
section 2.2, which prints a 1-bit quantizer: scale = (max - min) / (2**1 - 1),
zero_point = min, q = clamp(round((x - zero_point) / scale), 0, 1), with scale
and zero point returned as fp16.  The same section quantizes the key cache per
channel and the value cache per token; its section 5.2 asks for group sizes that
are multiples of 64.  The on-device KV article, section 3.1, gives INT4 keys
asymmetric per channel with a zero point and INT4 values in groups of 32/64.

Readings taken where the pages are silent or garbled:
  * b-bit generalization: the printed denominator 2**1 - 1 becomes 2**b - 1.
  * The printed code takes one min/max over its whole input; we take it per
    64-element group (the ``group_size`` argument it never uses).
  * Arithmetic: fp32 for max - min, the division and the code; the stored
    scale and zero point are fp16 (round to nearest even) and the code is
    computed against those stored fp16 values, so dequantization sees exactly
    what quantization assumed.  Rounding is half-to-even (``torch.round``).
  * A zero scale (all-equal group) yields code 0; the zero point then holds the
    value exactly.  Zeros are stored as +0.0: a -0.0 minimum, and the scale of
    a group of zeros of both signs (whose max - min could be -0.0 depending on
    which zero the reductions return).
  * Values are asymmetric for V as well (the printed quantizer and the stored
    zero point); the on-device article's "symmetric V" is not built.
  * A group is quantized only once all 64 of its tokens exist; until then its
    tokens stay fp16 (a "tail").  V follows K's group boundary.
  * The fp16 scale saturates: a range whose fp32 scale rounds past the largest
    finite fp16 (only possible at 1 bit, a range above 65504) stores 65504
    rather than infinity, so the codes stay 0/1 and every dequantized value is
    finite (the pages never meet such ranges; an infinite scale would turn the
    zero codes' products into NaN).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
GROUP = 64


def quantize_groups(x16: np.ndarray, bits: int):
    """Quantize each length-64 group along the last axis.

    x16: float16 array [..., 64].  Returns (codes uint8 [..., 64],
    scale float16 [...], zero float16 [...]).
    """
    assert x16.dtype == np.float16 and x16.shape[-1] == GROUP
    assert bits in (1, 4)
    levels = F32(2 ** bits - 1)
    x = x16.astype(F32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s32 = (mx - mn) / levels + F32(0.0)           # fp32, round to nearest even; +0 not -0
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    s16 = np.where(np.isinf(s16), np.float16(65504.0), s16)   # saturate (s32 >= 0)
    z16 = (mn + F32(0.0)).astype(np.float16)      # exact: mn is an fp16 value
    s = s16.astype(F32)[..., None]
    z = z16.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - z) / s                           # fp32 sub, fp32 div
    code = np.clip(np.rint(t), F32(0.0), levels)  # half to even
    code = np.where(s == 0, F32(0.0), code)
    return code.astype(np.uint8), s16, z16


def dequantize(code: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """code * scale + zero in fp64 (exact for fp16 scale/zero and codes < 16)."""
    return code.astype(np.float64) * s16.astype(np.float64) + z16.astype(np.float64)


def quantize_keys(k16: np.ndarray, bits: int):
    """Per-channel K quantization over complete 64-token groups.

    k16: float16 [N, D] for one (sequence, KV head).  Returns
    (codes uint8 [nq, D], scale f16 [nq/64, D], zero f16 [nq/64, D]) where
    nq = 64 * floor(N / 64); rows >= nq are the fp16 tail.
    """
    n, d = k16.shape
    ng = n // GROUP
    x = k16[: ng * GROUP].reshape(ng, GROUP, d).transpose(0, 2, 1)   # [ng, D, 64]
    code, s, z = quantize_groups(np.ascontiguousarray(x), bits)
    return code.transpose(0, 2, 1).reshape(ng * GROUP, d), s, z


def quantize_values(v16: np.ndarray, bits: int):
    """Per-token V quantization in 64-channel groups, over complete 64-token groups.

    v16: float16 [N, D].  Returns (codes uint8 [nq, D], scale f16 [nq, D/64],
    zero f16 [nq, D/64]).
    """
    n, d = v16.shape
    nq = (n // GROUP) * GROUP
    x = v16[:nq].reshape(nq, d // GROUP, GROUP)
    code, s, z = quantize_groups(np.ascontiguousarray(x), bits)
    return code.reshape(nq, d), s, z


def dequant_keys(code, s, z) -> np.ndarray:
    """fp64 K~ [nq, D] from per-channel group codes."""
    nq, d = code.shape
    rep_s = np.repeat(s, GROUP, axis=0)
    rep_z = np.repeat(z, GROUP, axis=0)
    return dequantize(code, rep_s, rep_z)


def dequant_values(code, s, z) -> np.ndarray:
    """fp64 V~ [nq, D] from per-token channel-group codes."""
    nq, d = code.shape
    rep_s = np.repeat(s, GROUP, axis=1)
    rep_z = np.repeat(z, GROUP, axis=1)
    return dequantize(code, rep_s, rep_z)


# ---------------------------------------------------------------------------
# Outlier channels.  Meeting-LLM article, section 8.2: after LayerNorm a very
# few channels carry values of very large magnitude; an offline analysis ranks
# each head's channels by their variance and marks the top ones as outliers;
# at run time the main cache holds the other channels quantized (with scale
# and zero point) and a separate store holds the outlier channels at their
# original precision; one fused kernel combines both into the full K vector.
# Readings taken:
#   * Variance: the population variance of each channel over the calibration
#     rows, compared exactly (fp16 values are integers times 2^-24, so
#     N * sum(x^2) - (sum x)^2 = N^2 * variance is an exact integer in those
#     units); ranking by (variance desc, channel asc); the list is returned
#     ascending.  The count is a parameter (0.5% of 128 channels is
#     less than one; the synthetic layers plant 3 outlier channels per head).
#   * One channel list per head serves K and V (the section isolates the
#     head's outlier channels for both); storing the V side is optional.
#   * In the main store an outlier channel's K scale and zero point are 0, so
#     its codes are 0 and it contributes nothing; its value comes from the
#     fp16 store instead.  V is grouped per token across channels: an outlier
#     channel is left out of its group's min/max and gets code 0; its value
#     comes from the fp16 store.
# ---------------------------------------------------------------------------

def outlier_channels(k16_calib: np.ndarray, m: int) -> np.ndarray:
    """The m channels of largest variance over the rows k16_calib [N, D], ascending."""
    x = np.asarray(k16_calib, dtype=np.float16).astype(np.float64) * 2.0 ** 24   # exact integers
    n, d = x.shape
    spread = []                                  # N^2 * variance per channel, exact
    for c in range(d):
        col = [int(v) for v in x[:, c]]
        spread.append(n * sum(v * v for v in col) - sum(col) ** 2)
    order = sorted(range(d), key=lambda c: (-spread[c], c))   # variance desc, channel asc
    return np.array(sorted(order[:m]), dtype=np.int32)


def quantize_keys_outliers(k16: np.ndarray, bits: int, out_ch: np.ndarray):
    """quantize_keys with the channels out_ch kept at fp16.

    Returns (codes, scale, zero, k_out) where codes/scale/zero are 0 on the
    outlier channels and k_out [nq, m] holds their fp16 values.
    """
    code, s, z = quantize_keys(k16, bits)
    ch = np.asarray(out_ch, dtype=np.int64)
    code[:, ch] = 0
    s[:, ch] = np.float16(0.0)
    z[:, ch] = np.float16(0.0)
    k_out = np.ascontiguousarray(k16[: code.shape[0]][:, ch])
    return code, s, z, k_out


def quantize_values_outliers(v16: np.ndarray, bits: int, out_ch: np.ndarray):
    """quantize_values with the channels out_ch left out of every group's range.

    Each outlier entry is replaced by the smallest of its group's other values
    (which leaves min and max those of the other channels and gives code 0),
    then the groups are quantized as usual.  Returns (codes, scale, zero, v_out)
    with v_out [nq, m] the outlier channels' fp16 values.
    """
    n, d = v16.shape
    nq = (n // GROUP) * GROUP
    ch = np.asarray(out_ch, dtype=np.int64)
    x = v16[:nq].copy()
    other = np.ones(d, bool)
    other[ch] = False
    for h in range(d // GROUP):
        cols = np.arange(h * GROUP, (h + 1) * GROUP)
        mine = ch[(ch >= h * GROUP) & (ch < (h + 1) * GROUP)]
        if len(mine) and nq:
            low = x[:, cols[other[cols]]].min(axis=1)
            x[:, mine] = low[:, None]
    code, s, z = quantize_values(x, bits)
    code[:, ch] = 0
    v_out = np.ascontiguousarray(v16[:nq][:, ch])
    return code, s, z, v_out


def dequant_values_outliers(code, s, z, out_ch, v_out) -> np.ndarray:
    """fp64 V~ [nq, D]: dequantized codes, with the outlier channels' fp16 values."""
    v = dequant_values(code, s, z)
    v[:, np.asarray(out_ch, dtype=np.int64)] = v_out.astype(np.float64)
    return v


def dequant_keys_outliers(code, s, z, out_ch, k_out) -> np.ndarray:
    """fp64 K~ [nq, D]: dequantized codes, with the outlier channels' fp16 values."""
    k = dequant_keys(code, s, z)
    k[:, np.asarray(out_ch, dtype=np.int64)] = k_out.astype(np.float64)
    return k


# ---------------------------------------------------------------------------
# FP8 (E4M3) warm tier.  Meeting-LLM article, section 6.2: the warm (L2) tier
# prefers FP8 E4M3/E5M2 over INT4 where the hardware supports it natively; KV
# compression survey, section 2: an FP8 E4M3/E5M2 KV cache halves memory and
# doubles bandwidth without reworking the dequantization.
# Readings taken:
#   * E4M3 as the OCP 8-bit format: 1 sign, 4 exponent (bias 7), 3 mantissa
#     bits, subnormals, no infinities, largest finite 448.
#   * A plain per-element cast (no scale: the pages need no new dequantization),
#     round to nearest with ties to the even code, saturating at +-448; the sign
#     of zero is kept.
#   * Every token is encoded when appended (no groups, no fp16 tail).
# ---------------------------------------------------------------------------

def _fp8_magnitudes() -> np.ndarray:
    """Exact value of every non-negative finite E4M3 code 0x00..0x7E (index = code)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals, dtype=np.float64)


FP8_MAG = _fp8_magnitudes()


def encode_fp8(x16: np.ndarray) -> np.ndarray:
    """fp16 -> E4M3 code: the nearest grid value, ties to the even code, saturating.

    The two grid magnitudes around |x| are compared (exact in fp64: every fp16
    and every E4M3 value is a short dyadic rational).
    """
    x = np.asarray(x16, dtype=np.float16)
    assert np.all(np.isfinite(x))
    a = np.abs(x.astype(np.float64)).reshape(-1)
    hi = np.minimum(np.searchsorted(FP8_MAG, a), 0x7E)        # first magnitude >= |x| (capped)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - FP8_MAG[lo]
    d_hi = FP8_MAG[hi] - a
    pick = np.where(d_hi < d_lo, hi, lo)
    pick = np.where(d_hi == d_lo, np.where(hi % 2 == 0, hi, lo), pick)   # tie: the even code
    pick = np.where(a >= FP8_MAG[-1], 0x7E, pick)             # 448 and beyond: saturate
    sign = np.signbit(x).reshape(-1).astype(np.int64) << 7
    return (pick | sign).astype(np.uint8).reshape(x.shape)


def decode_fp8(code: np.ndarray) -> np.ndarray:
    """E4M3 code -> exact value (fp64)."""
    c = np.asarray(code, dtype=np.int64)
    mag = FP8_MAG[np.minimum(c & 0x7F, 0x7E)]
    return np.where(c & 0x80, -mag, mag)
