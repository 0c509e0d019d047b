"""GPU parity of kvc_quantize_append against the oracle: codes, scales, zeros,
tails, fp16 copies and max|K| bit-exact, over ragged multi-step appends,
contiguous and paged caches, and the full-size 128K / 32K prefill."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import KvcCache
from gpu_util import dev, host
from kvc_layout import slots, unpack_codes
from oracle import step as ST

pytestmark = pytest.mark.gpu


def _u16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def check_cache_state(cache: KvcCache, rows_k, rows_v, lens, table=None):
    """Compare every buffer of ``cache`` with the oracle's cache for rows[:len]."""
    fmt = cache.fmt
    seq = host(cache.seq_lens)
    assert seq.tolist() == list(lens), (seq, lens)
    absmax = host(cache.k_absmax)
    if fmt != "fp16":
        kc, vc = host(cache.k_codes), host(cache.v_codes)
        km, vm = host(cache.k_meta), host(cache.v_meta)
        kt, vt = host(cache.k_tail), host(cache.v_tail)
    k16 = host(cache.k16) if cache.k16 is not None else None
    v16 = host(cache.v16) if cache.v16 is not None else None
    kT = host(cache.kT) if cache.kT is not None else None
    for b in range(cache.batch):
        n = int(lens[b])
        for g in range(cache.hkv):
            hc = ST.build_head_cache(rows_k[b][:n, g], rows_v[b][:n, g], fmt)
            where = f"b={b} g={g} n={n}"
            assert np.array_equal(_u16(absmax[b, g].astype(np.float16)), _u16(hc.kabs)), where
            sl = slots(b, g, np.arange(n), cache.hkv, cache.max_tokens, cache.page_size, table)
            if k16 is not None:
                assert np.array_equal(_u16(k16[sl]), _u16(hc.k16)), where
                assert np.array_equal(_u16(v16[sl]), _u16(hc.v16)), where
            if kT is not None:
                assert np.array_equal(_u16(kT[b, g, :, :n].T), _u16(hc.k16)), where
            if fmt == "fp16":
                continue
            nq = hc.nq
            sq = sl[:nq]
            assert np.array_equal(unpack_codes(kc, fmt, "k", sq), hc.k_code), "K codes " + where
            assert np.array_equal(unpack_codes(vc, fmt, "v", sq), hc.v_code), "V codes " + where
            assert np.array_equal(_u16(km[b, g, : nq // 64, 0]), _u16(hc.k_scale)), where
            assert np.array_equal(_u16(km[b, g, : nq // 64, 1]), _u16(hc.k_zero)), where
            assert np.array_equal(_u16(vm[sq, 0:2]), _u16(hc.v_scale)), where
            assert np.array_equal(_u16(vm[sq, 2:4]), _u16(hc.v_zero)), where
            assert np.array_equal(_u16(kt[b, g, : n - nq]), _u16(hc.k16[nq:])), "tail " + where
            assert np.array_equal(_u16(vt[b, g, : n - nq]), _u16(hc.v16[nq:])), "tail " + where


def _rows(rng, B, n, hkv, outliers=True):
    k = rng.standard_normal((B, n, hkv, 128), dtype=np.float32)
    if outliers:
        k[..., [3, 77]] *= 8
    v = rng.standard_normal((B, n, hkv, 128), dtype=np.float32)
    k[0, :64, 0, 5] = 0.0            # an all-equal channel group (zero scale)
    v[0, 7, 0, :64] = -1.25          # an all-equal value group
    return k.astype(np.float16), v.astype(np.float16)


STEPS = [[100, 64, 3], [1, 1, 1], [63, 0, 130], [70, 5, 61], [1, 64, 0]]


# (complete groups of new rows on a cache without fp16 rows or outliers take
# the quantizer's direct-load mode, the others the staged one: both run here)
@pytest.mark.parametrize("fmt,page,rows", [("int4", 0, False), ("int1", 0, False), ("int4", 16, True),
                                           ("int1", 64, False), ("int4", 32, False), ("int4", 16, False),
                                           ("fp16", 0, True), ("fp16", 16, True)])
def test_incremental_ragged_appends(fmt, page, rows):
    rng = np.random.default_rng(7)
    B, hkv, cap = 3, 2, 384
    total = np.sum(STEPS, axis=0)
    k, v = _rows(rng, B, int(total.max()), hkv)
    table = None
    kw = {}
    if page:
        per = cap // page
        table = rng.permutation(B * per).astype(np.int32).reshape(B, per)
        kw = dict(page_size=page, block_table=torch.from_numpy(table), num_pages=B * per)
    cache = KvcCache(fmt, B, hkv, cap, fp16_rows=rows, kT=(fmt == "fp16" and page == 0), **kw)
    lens = np.zeros(B, np.int64)
    for step in STEPS:
        nmax = max(step)
        kn = np.zeros((B, nmax, hkv, 128), np.float16)
        vn = np.zeros_like(kn)
        for b in range(B):
            kn[b, :step[b]] = k[b, lens[b]:lens[b] + step[b]]
            vn[b, :step[b]] = v[b, lens[b]:lens[b] + step[b]]
        cache.append(dev(kn), dev(vn), dev(np.array(step, np.int32)))
        lens += step
        torch.cuda.synchronize()
        check_cache_state(cache, k, v, lens, table)


def test_overflow_leaves_sequence_unchanged():
    rng = np.random.default_rng(8)
    k, v = _rows(rng, 2, 128, 1)
    cache = KvcCache("int4", 2, 1, 128)
    cache.append(dev(k[:, :100]), dev(v[:, :100]))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kn = np.concatenate([k[:, 100:128], k[:, :10]], axis=1)
    vn = np.concatenate([v[:, 100:128], v[:, :10]], axis=1)
    n_new = dev(np.array([38, 28], np.int32))     # sequence 0 would reach 138 > 128
    cache.append(dev(kn), dev(vn), n_new, overflow=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    rows_k = [k[0], np.concatenate([k[1, :100], kn[1, :28]])]
    rows_v = [v[0], np.concatenate([v[1, :100], vn[1, :28]])]
    check_cache_state(cache, rows_k, rows_v, [100, 128])


def _check_fp8_rows(cache: KvcCache, rows_k, rows_v, lens, table=None):
    from oracle import quant as Q
    assert host(cache.seq_lens).tolist() == list(lens)
    kc = host(cache.k_codes).reshape(-1, 128)
    vc = host(cache.v_codes).reshape(-1, 128)
    for b in range(cache.batch):
        n = int(lens[b])
        for g in range(cache.hkv):
            sl = slots(b, g, np.arange(n), cache.hkv, cache.max_tokens, cache.page_size, table)
            assert np.array_equal(kc[sl], Q.encode_fp8(rows_k[b][:n, g])), (b, g)
            assert np.array_equal(vc[sl], Q.encode_fp8(rows_v[b][:n, g])), (b, g)


@pytest.mark.parametrize("fmt,page", [("int4", 0), ("int1", 0), ("int4", 16), ("int1", 64),
                                      ("fp16", 0), ("fp8", 16)])
def test_single_token_steps(fmt, page):
    """One-token appends (one launch per step) from ragged lengths across group
    boundaries, with n_new absent and with n_new holding zeros: every buffer
    equals the oracle's cache after each few steps, for 5 KV heads."""
    rng = np.random.default_rng(40)
    B, hkv, cap, steps = 3, 5, 256, 70
    start = np.array([60, 0, 127], np.int64)
    k, v = _rows(rng, B, int(start.max()) + steps, hkv)
    table, kw = None, {}
    if page:
        per = cap // page
        table = rng.permutation(B * per).astype(np.int32).reshape(B, per)
        kw = dict(page_size=page, block_table=torch.from_numpy(table), num_pages=B * per)
    cache = KvcCache(fmt, B, hkv, cap, fp16_rows=fmt == "fp16" or (fmt != "fp8" and page == 16),
                     kT=(fmt == "fp16"), **kw)
    check = _check_fp8_rows if fmt == "fp8" else check_cache_state
    cache.append(dev(k[:, :int(start.max())]), dev(v[:, :int(start.max())]),
                 dev(start.astype(np.int32)))
    lens = start.copy()
    for i in range(steps):
        step = np.ones(B, np.int64) if i % 3 == 0 else rng.integers(0, 2, size=B)
        kn = np.zeros((B, 1, hkv, 128), np.float16)
        vn = np.zeros_like(kn)
        for b in range(B):
            if step[b]:
                kn[b, 0], vn[b, 0] = k[b, lens[b]], v[b, lens[b]]
        cache.append(dev(kn), dev(vn), None if i % 3 == 0 else dev(step.astype(np.int32)))
        lens += step
        if i % 10 == 9 or i == steps - 1:
            torch.cuda.synchronize()
            check(cache, k, v, lens, table)


def test_single_token_overflow():
    """A one-token append to a full sequence, or with n_new[b] above n_new_max = 1,
    sets the flag and leaves that sequence as it was; the others grow."""
    rng = np.random.default_rng(41)
    B, hkv, cap = 3, 3, 128
    k, v = _rows(rng, B, cap + 2, hkv)
    cache = KvcCache("int4", B, hkv, cap)
    start = np.array([128, 100, 63], np.int32)
    cache.append(dev(k[:, :128]), dev(v[:, :128]), dev(start))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kn = np.stack([k[b, start[b] % cap] for b in range(B)])[:, None]
    vn = np.stack([v[b, start[b] % cap] for b in range(B)])[:, None]
    cache.append(dev(kn), dev(vn), overflow=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    rows_k = [k[0, :128], k[1, :101], k[2, :64]]
    rows_v = [v[0, :128], v[1, :101], v[2, :64]]
    check_cache_state(cache, rows_k, rows_v, [128, 101, 64])
    flag.zero_()
    kn2 = np.stack([k[0, 0], k[1, 101], k[2, 64]])[:, None]
    vn2 = np.stack([v[0, 0], v[1, 101], v[2, 64]])[:, None]
    cache.append(dev(kn2), dev(vn2), dev(np.array([0, 2, 1], np.int32)), overflow=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    rows_k[2] = k[2, :65]
    rows_v[2] = v[2, :65]
    check_cache_state(cache, rows_k, rows_v, [128, 101, 65])


@pytest.mark.parametrize("make", [lambda: W.int1_dense(131072), lambda: W.int4_dense(32768)],
                         ids=["int1_128k", "int4_32k"])
def test_full_size_prefill(make):
    w = make()
    cache = KvcCache(w.fmt, w.batch, w.hkv, w.max_tokens)
    cache.append(dev(w.k), dev(w.v))
    torch.cuda.synchronize()
    check_cache_state(cache, w.k, w.v, w.seq_lens)


@pytest.mark.parametrize("fmt,rows", [("int4", False), ("int1", False), ("int4", True), ("int1", True)])
def test_code_rounding_at_half_integers(fmt, rows):
    """Values whose quotient (x - z) / s is exactly a half-integer, or one fp16 step
    off it, for scales with inexact reciprocals (3, 7, 0.75, 5/16, ...): the
    kernel's codes (a reciprocal product, the division near half-integers) equal
    the oracle's correctly rounded quotient, ties to even, for K channels and V rows
    (without fp16 rows the groups take the direct-load quantizer, with them the
    staged one)."""
    top = 15 if fmt == "int4" else 1
    rng = np.random.default_rng(50)
    hkv = 2
    k = rng.standard_normal((1, 128, hkv, 128)).astype(np.float16)
    v = rng.standard_normal((1, 128, hkv, 128)).astype(np.float16)
    scales = [1.0, 3.0, 7.0, 0.75, 0.3125, 5.0, 6.0, 0.1875, 11.0, 13.0, 0.0390625]
    for ci, sc in enumerate(scales):
        for grp in range(2):
            z = float(np.float16(-2.0 * (ci + 1) + grp))
            col = [z, z + top * sc]
            for kk in range(top):
                h = np.float16(z + (kk + 0.5) * sc)
                col += [float(h), float(np.nextafter(h, np.float16(np.inf))),
                        float(np.nextafter(h, np.float16(-np.inf)))]
            col = np.resize(np.array(col, np.float32), 64).astype(np.float16)
            for g in range(hkv):
                k[0, 64 * grp:64 * grp + 64, g, ci] = col             # a K channel over the group
                v[0, 64 * grp + ci, g, :64] = col                     # a V row, low half
                v[0, 64 * grp + ci, g, 64:] = col[::-1]               # and high half
    cache = KvcCache(fmt, 1, hkv, 192, fp16_rows=rows)
    cache.append(dev(k), dev(v))
    torch.cuda.synchronize()
    check_cache_state(cache, k, v, [128])


def test_one_bit_scale_saturates():
    """1-bit groups whose range exceeds 65504 (K per channel and V per token) store the
    saturated scale 65504 as the oracle does, and attention over them stays finite."""
    from decode_attention_sparse_kvc_amd import kvc
    rng = np.random.default_rng(30)
    k, v = _rows(rng, 1, 128, 1, outliers=False)
    k[0, :64, 0, 9] = np.linspace(-40000, 40000, 64).astype(np.float16)   # one K channel group
    v[0, 70, 0, :64] = np.linspace(-33000, 33000, 64).astype(np.float16)  # one V token group
    cache = KvcCache("int1", 1, 1, 192)
    cache.append(dev(k), dev(v))
    torch.cuda.synchronize()
    check_cache_state(cache, k, v, [128])
    assert host(cache.k_meta)[0, 0, 0, 0, 9] == np.float16(65504.0)
    q = dev(rng.standard_normal((1, 1, 128)).astype(np.float16) * np.float16(1e-5))
    out = torch.empty(1, 1, 128, device="cuda")
    lse = torch.empty(1, 1, device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, 1)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    kvc.kvc_attend_decode(cache.desc, q, 1, 128 ** -0.5, 0, None, 0, 0, 0, out, lse, None, 0, ws, nb)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(out))) and np.all(np.isfinite(host(lse)))
