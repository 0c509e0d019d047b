"""GPU parity of INT4 caches with outlier channels kept at fp16 (meeting-LLM
article, section 8.2; K, and V unless its store is absent): main-store codes,
scales, zeros and the outlier stores bit for bit against the oracle; scores and Top-K bit for bit; attention (dense,
drop, keep, blocks; contiguous and paged) within 1e-3 + 2e-3 |ref|, including
the 128K layer."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import KvcCache
from gpu_util import assert_close, cache_for, dev, host, prefill
from kvc_layout import slots, unpack_codes
from oracle import quant as Q
from oracle import step as ST
from test_gpu_attend import check_against_oracle, oracle_and_cache, paged, run_attend, sel_tensor
from test_gpu_blocks import block_case
from test_gpu_topk import topk_case

pytestmark = pytest.mark.gpu


def _u16(a):
    return np.ascontiguousarray(a).view(np.uint16)


@pytest.mark.parametrize("page,m", [(0, 3), (16, 1), (64, 4)])
def test_store_after_ragged_appends(page, m):
    """Two sequences appended in ragged steps (groups completed by prefill-sized
    and single-token appends): main store and outlier store equal the oracle's."""
    rng = np.random.default_rng(31 + m)
    B, hkv, cap = 2, 2, 384
    ch = np.stack([np.sort(rng.choice(128, m, replace=False)) for _ in range(hkv)]).astype(np.int32)
    table, npages = None, 0
    if page:
        per = cap // page
        npages = B * per
        table = rng.permutation(npages).astype(np.int32).reshape(B, per)
    cache = KvcCache("int4", B, hkv, cap, page_size=page,
                     block_table=None if table is None else torch.from_numpy(table),
                     num_pages=npages, outlier_ch=torch.from_numpy(ch))
    rows_k = [np.zeros((0, hkv, 128), np.float16) for _ in range(B)]
    rows_v = [np.zeros((0, hkv, 128), np.float16) for _ in range(B)]
    for step, n_new in enumerate([[130, 64], [1, 63], [62, 1], [1, 1]]):
        n_new = np.array(n_new, np.int32)
        mx = int(n_new.max())
        k = rng.normal(size=(B, mx, hkv, 128)).astype(np.float32)
        v = rng.normal(size=(B, mx, hkv, 128)).astype(np.float32)
        for g in range(hkv):
            k[:, :, g, ch[g]] *= 20.0
            v[:, :, g, ch[g]] *= 30.0
        k = k.astype(np.float16)
        v = v.astype(np.float16)
        cache.append(dev(k), dev(v), dev(n_new))
        for b in range(B):
            rows_k[b] = np.concatenate([rows_k[b], k[b, : n_new[b]]])
            rows_v[b] = np.concatenate([rows_v[b], v[b, : n_new[b]]])
    torch.cuda.synchronize()
    kc, km, ko = host(cache.k_codes), host(cache.k_meta), host(cache.k_outlier)
    vc, vm, vo = host(cache.v_codes), host(cache.v_meta), host(cache.v_outlier)
    for b in range(B):
        n = rows_k[b].shape[0]
        for g in range(hkv):
            hc = ST.build_head_cache(rows_k[b][:, g], rows_v[b][:, g], "int4", ch[g])
            nq = hc.nq
            sl = slots(b, g, np.arange(nq), hkv, cap, page, table)
            where = f"b={b} g={g} n={n}"
            assert np.array_equal(unpack_codes(kc, "int4", "k", sl), hc.k_code), "K codes " + where
            assert np.array_equal(_u16(km[b, g, : nq // 64, 0]), _u16(hc.k_scale)), where
            assert np.array_equal(_u16(km[b, g, : nq // 64, 1]), _u16(hc.k_zero)), where
            assert np.array_equal(_u16(ko[sl, :m]), _u16(hc.k_out)), "outlier store " + where
            assert not _u16(ko[sl, m:]).any(), where
            assert np.array_equal(unpack_codes(vc, "int4", "v", sl), hc.v_code), "V codes " + where
            assert np.array_equal(_u16(vm[sl, 0:2]), _u16(hc.v_scale)), where
            assert np.array_equal(_u16(vm[sl, 2:4]), _u16(hc.v_zero)), where
            assert np.array_equal(_u16(vo[sl, :m]), _u16(hc.v_out)), "V outlier store " + where
            assert not _u16(vo[sl, m:]).any(), where


@pytest.mark.parametrize("n", [63, 777, 4095, 4097])
def test_dense(n):
    """Prefill n tokens, append the step's token (4095 + 1 completes a group on the
    single-token path), attend over everything."""
    w = W.int4_outlier_dense(n)
    res = ST.decode_step(w, append=True, pairs=[(0, 0), (0, 3), (0, 7)])
    cache = cache_for(w)
    prefill(cache, w)
    cache.append(dev(w.k_new), dev(w.v_new))
    out, lse, lg, _ = run_attend(cache, w)
    G = w.group
    for (b, g), toks in res.tokens.items():
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")
        assert_close(lg[b, sl][:, toks], res.logits[(b, g)], f"logits g={g}")


@pytest.mark.parametrize("outlier_v", [False, True])
def test_dense_value_outliers(outlier_v):
    """V channels scaled x30 on the outlier list: with the V store their output is
    the fp16 values' (the codes' group zero replaced); without it (K only) V is
    quantized with the outliers in range."""
    w = W.int4_outlier_dense(2000)
    w.v = w.v.astype(np.float32)
    for g in range(w.hkv):
        w.v[:, :, g, w.outlier_ch[g]] *= 30.0
    w.v = w.v.astype(np.float16)
    w.outlier_v = outlier_v
    res = ST.decode_step(w, append=True, pairs=[(0, 1), (0, 4)])
    cache = cache_for(w)
    assert (cache.v_outlier is not None) == outlier_v
    prefill(cache, w)
    cache.append(dev(w.k_new), dev(w.v_new))
    out, lse, lg, _ = run_attend(cache, w)
    G = w.group
    for (b, g), toks in res.tokens.items():
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")


@pytest.mark.parametrize("page", [16, 32, 64])
def test_dense_paged(page):
    w = paged(W.int4_outlier_dense(3000), page, seed=page)
    res = ST.decode_step(w, append=False, pairs=[(0, 1), (0, 6)])
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, _, _ = run_attend(cache, w, logits=False)
    G = w.group
    for (b, g) in res.tokens:
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")


def test_exact_topk_single_head():
    """The 4K single-head case with its 4 outlier channels found by the offline
    variance analysis: exact scores (which read the outlier store) and indices bit
    for bit, then drop-mode attention over sinks + Top-128 + window."""
    w = W.single_head_4k(2000)
    w.outlier_ch = Q.outlier_channels(w.k[0, :, 0], 4)[None]
    res, cache, idx = topk_case(w, append=True)
    km = int(w.top_k.max())
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, km), km)
    check_against_oracle(w, res, out, lse, lg, km, stride)


def test_critical_topk_drop():
    """Critical channels on an INT4 layer whose outlier channels are the planted
    ones: scores, channels and indices bit for bit, attention in tolerance."""
    w = W.sparse_crit8(n_ctx=3000, n_planted=40, top_k=200)
    w.fmt = "int4"
    w.outlier_ch = np.stack([Q.outlier_channels(w.k[0, :, g], 2) for g in range(w.hkv)])
    res, cache, idx = topk_case(w)
    km = int(w.top_k.max())
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, km), km)
    check_against_oracle(w, res, out, lse, lg, km, stride)


def test_full_size_dense():
    """The 128K INT4 layer with its 3 outlier channels per KV head, in the
    benchmark's launch configuration, sampled pairs."""
    w = W.FULL["llama8b_layer_int4_outlier3_dense_128k"]()
    res = ST.decode_step(w, append=True, pairs=[(0, 2), (0, 5)])
    cache = cache_for(w)
    prefill(cache, w)
    cache.append(dev(w.k_new), dev(w.v_new))
    out, lse, _, _ = run_attend(cache, w, logits=False)
    G = w.group
    for (b, g) in res.tokens:
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")


@pytest.mark.parametrize("append", [False, True])
def test_keep_paged_ragged(append):
    """Joint tiers on 16-token pages with outlier channels: the keep set in fp16,
    the rest from the codes plus the outlier store, H2O-ranked keep set."""
    w = W.batched_joint(batch=3, lo=500, hi=900, n_window=128)
    rng = np.random.default_rng(5)
    w.outlier_ch = np.stack([np.sort(rng.choice(128, 3, replace=False)) for _ in range(w.hkv)]).astype(np.int32)
    res, cache = oracle_and_cache(w, append=append)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    k_max = int(w.top_k.max())
    out, lse, lg, _ = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg)


def test_blocks_critical():
    """Block-granular selection on an INT4 layer with outlier channels: block means
    (from scores that read the outlier store) and kept blocks bit for bit, then
    blocks-mode attention."""
    w = W.sparse_blocks(n_ctx=3000, fmt="int4", top_blocks=7)
    w.n_sink, w.n_window = 4, 200
    w.outlier_ch = np.stack([Q.outlier_channels(w.k[0, :, g], 2) for g in range(w.hkv)])
    block_case(w, append=True, pairs=[(0, 2), (0, 4)])


@pytest.mark.parametrize("G,page", [(1, 0), (2, 16), (8, 0), (8, 32)])
def test_group_sizes(G, page):
    """Query groups of 1, 2 and 8 heads (8: the unpacked softmax path), with planted
    K and V outliers on the list, contiguous and paged."""
    w = W.int4_dense(900)
    w.hkv = 32 // G if G < 8 else 4
    w.hq = w.hkv * G
    rng = np.random.default_rng(40 + G)
    k = rng.standard_normal((1, 900, w.hkv, 128), dtype=np.float32)
    v = rng.standard_normal((1, 900, w.hkv, 128), dtype=np.float32)
    w.outlier_ch = np.stack([np.sort(rng.choice(128, 3, replace=False)) for _ in range(w.hkv)]).astype(np.int32)
    for g in range(w.hkv):
        k[:, :, g, w.outlier_ch[g]] *= 16.0
        v[:, :, g, w.outlier_ch[g]] *= 16.0
    w.k, w.v = k.astype(np.float16), v.astype(np.float16)
    w.q = rng.standard_normal((1, w.hq, 128), dtype=np.float32).astype(np.float16)
    if page:
        paged(w, page, seed=G)
    res, cache = oracle_and_cache(w)
    out, lse, lg, _ = run_attend(cache, w)
    check_against_oracle(w, res, out, lse, lg)
