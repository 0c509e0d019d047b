"""Reading the library's packed buffers back into logical arrays, from include/kvc.h's text.

Test infrastructure: written from the header's layout description, shares no
code with the HIP kernels and none with the oracle.
"""
from __future__ import annotations

import numpy as np


def slots(b: int, g: int, t: np.ndarray, hkv: int, max_tokens: int, page_size: int,
          table: np.ndarray | None) -> np.ndarray:
    """slot = (phys * Hkv + g) * P + t % P  (int64)."""
    t = np.asarray(t, dtype=np.int64)
    P = page_size if page_size > 0 else max_tokens
    if page_size > 0:
        phys = table[b, t // P].astype(np.int64)
    else:
        phys = np.full_like(t, b)
    return (phys * hkv + g) * P + t % P


def nib_pos(j):
    j = np.asarray(j)
    return 16 * (j & 1) + 4 * (j >> 1)


def bit_pos(k):
    k = np.asarray(k)
    w, h = k >> 1, k & 1
    v, p = w >> 2, 6 + (w & 3)
    return np.where(v == 0, p + 16 * h,
           np.where(v == 1, p + 4 + 16 * h,
           np.where(v == 2, p - 4 + 16 * h,
                    np.where(h == 1, p + 8, (p + 24) & 31))))


def v1_code(ct, i):
    ct, i = np.asarray(ct), np.asarray(i)
    return 2 * (4 * ((ct >> 2) * 2 + (i >> 1)) + (ct & 3)) + (i & 1)


def unpack_codes(buf: np.ndarray, fmt: str, which: str, slot: np.ndarray) -> np.ndarray:
    """Logical codes [T, 128] of the tokens at ``slot`` (their offsets inside a
    tile/unit are slot % 16 or slot % 64, as the header's tiling implies)."""
    words = buf.view(np.uint32)
    c = np.arange(128)[None, :]
    s = slot[:, None]
    if fmt == "int4":
        tile, n = s // 16, s % 16
        if which == "k":
            lane, d, j = 16 * (c // 32) + n, (c % 32) // 8, c % 8
        else:
            lane, d, j = 16 * (n // 4) + c % 16, (c // 16) // 2, 4 * ((c // 16) % 2) + n % 4
        u = words[tile * 256 + lane * 4 + d]
        return ((u >> nib_pos(j).astype(np.uint32)) & 15).astype(np.uint8)
    unit, n = s // 64, s % 64
    if which == "k":
        lane, d, k = 16 * (c // 32) + n % 16, n // 16, c % 32
    else:
        lane, d, k = 16 * ((n % 16) // 4) + c % 16, n // 16, v1_code(c // 16, n % 4)
    u = words[unit * 256 + lane * 4 + d]
    return ((u >> bit_pos(k).astype(np.uint32)) & 1).astype(np.uint8)


def check_bit_tables():
    """Every INT1 dword bit is used exactly once; every INT4 nibble slot once."""
    assert sorted(bit_pos(np.arange(32)).tolist()) == list(range(32))
    assert sorted(nib_pos(np.arange(8)).tolist()) == list(range(0, 32, 4))
    ks = sorted(int(v1_code(ct, i)) for ct in range(8) for i in range(4))
    assert ks == list(range(32))
