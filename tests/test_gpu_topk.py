"""GPU parity of kvc_score_topk and kvc_accum_scores against the oracle.

Critical channels, per-token fp64 scores and Top-K indices must match bit for
bit (the interface fixes the summation order); H2O accumulators within
1e-3 + 2e-3 |ref|.  Covers exact / critical / external modes on fp16 (with and
without the channel-major copy, contiguous and paged), INT4 and 1-bit caches,
planted ties, ragged k, empty candidate ranges and the full-size workloads.
"""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import step as ST
from test_gpu_attend import run_attend, sel_tensor

pytestmark = pytest.mark.gpu


def run_topk(cache, w, k_max=None, scores=True):
    B, hkv = w.batch, w.hkv
    k_max = int(w.top_k.max()) if k_max is None else k_max
    idx = torch.full((B, hkv, max(k_max, 1)), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, hkv, cache.max_tokens), float("nan"), dtype=torch.float64, device="cuda") if scores else None
    ch = torch.full((B, hkv, w.n_crit), -7, dtype=torch.int32, device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, cache.desc, w.hq)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ext = dev(w.acc) if w.score == "external" else None
    kps = dev(w.top_k.astype(np.int32))
    kvc.kvc_score_topk(cache.desc, dev(w.q), w.hq, kvc.SCORE[w.score], w.n_crit, ext, w.n_sink,
                       w.n_window, kps, k_max, idx, sc, ch, ws, nb)
    torch.cuda.synchronize()
    return host(idx)[:, :, :k_max], (host(sc) if scores else None), host(ch)


def check_topk(w, res, idx, sc, ch, k_max):
    for (b, g), ref_sel in res.sel.items():
        n = res.caches[(b, g)].n
        lo, hi = w.n_sink, n - w.n_window
        where = f"b={b} g={g}"
        if w.score == "critical":
            assert ch[b, g].tolist() == res.channels[(b, g)].tolist(), "channels " + where
        if sc is not None and hi > lo:
            got = sc[b, g, lo:hi]
            ref = res.scores[(b, g)][lo:hi]
            assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), "scores " + where
        want = np.full(k_max, -1, np.int64)
        want[: len(ref_sel)] = ref_sel[:k_max]
        assert np.array_equal(idx[b, g], want), f"indices {where}: {idx[b, g][:12]} vs {want[:12]}"


def topk_case(w, append=False, k_max=None):
    res = ST.decode_step(w, append=append, k_max=k_max)
    cache = cache_for(w)
    prefill(cache, w)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    km = int(w.top_k.max()) if k_max is None else k_max
    idx, sc, ch = run_topk(cache, w, km)
    check_topk(w, res, idx, sc, ch, km)
    return res, cache, idx


@pytest.mark.parametrize("n", [3000, 4097])
def test_critical_fp16_channel_major(n):
    w = W.sparse_crit8(n_ctx=n, n_planted=60, top_k=300)
    topk_case(w)


@pytest.mark.parametrize("page", [0, 16])
def test_critical_fp16_rows(page):
    w = W.sparse_crit8(n_ctx=2000, n_planted=40, top_k=150)
    w.kT = False
    if page:
        per = w.max_tokens // page
        w.page_size, w.num_pages = page, per
        w.block_table = np.random.default_rng(3).permutation(per).astype(np.int32)[None]
    topk_case(w)


@pytest.mark.parametrize("n", [1000, 4096])
def test_exact_int4_single_head(n):
    topk_case(W.single_head_4k(n))


def test_exact_int4_single_head_long():
    """One pair of 200K tokens with exact scores: more counting workgroups than histogram
    slots would allow, so the scoring grid is capped (256 slots) and each workgroup loops
    over several chunks; the long-range path (compaction, regions) selects."""
    w = W.single_head_4k(200_000)
    w.top_k = np.array([3000], np.int32)
    topk_case(w)


def test_exact_int4_after_append():
    topk_case(W.single_head_4k(700), append=True)


@pytest.mark.parametrize("score", ["exact", "critical"])
def test_int1_scores(score):
    w = W.int1_dense(1500)
    w.score, w.mode, w.top_k, w.n_sink, w.n_window = score, "drop", np.array([100], np.int32), 4, 64
    topk_case(w)


def test_external_ragged_k():
    w = W.batched_joint(batch=4, lo=400, hi=900, n_window=128)
    topk_case(w)


def test_planted_ties():
    """Many exactly equal scores: the lower token index wins at the boundary."""
    w = W.sparse_crit8(n_ctx=1200, n_planted=0, top_k=77)
    k = w.k.copy()
    for g in range(w.hkv):           # 200 identical rows per KV head, scoring far above the rest
        k[0, 100:700:3, g] = (2 * w.q[0, 4 * g].astype(np.float32)).astype(np.float16)
    w.k = k
    w.n_crit = 128                    # exact score over every channel -> identical scores
    topk_case(w)
    w.score = "exact"
    topk_case(w)


@pytest.mark.parametrize("k_max,top", [(1, 1), (64, 0), (64, 5000), (300, 300)])
def test_k_edges(k_max, top):
    w = W.sparse_crit8(n_ctx=900, n_planted=10, top_k=top)
    topk_case(w, k_max=k_max)


def test_no_candidates():
    w = W.sparse_crit8(n_ctx=100, n_planted=4, top_k=10)
    w.n_sink, w.n_window = 60, 60
    res, cache, idx = topk_case(w, k_max=10)
    assert np.all(idx == -1)


def test_sixteen_heads_per_kv_head():
    w = W.sparse_crit8(n_ctx=800, n_planted=10, top_k=40)
    w.hkv = 2
    rng = np.random.default_rng(6)
    w.k = rng.standard_normal((1, 800, 2, 128), dtype=np.float32).astype(np.float16)
    w.v = rng.standard_normal((1, 800, 2, 128), dtype=np.float32).astype(np.float16)
    topk_case(w)


def test_region_path_ties_across_regions():
    """Above 8192 items each 4096-item region emits its own indices: identical scores spread
    over five regions, the selection boundary among them (lower index wins across regions)."""
    w = W.sparse_crit8(n_ctx=20000, n_planted=0, top_k=500)
    k = w.k.copy()
    for g in range(w.hkv):           # ~610 identical rows per KV head, scoring far above the rest
        k[0, 100:19000:31, g] = (2 * w.q[0, 4 * g].astype(np.float32)).astype(np.float16)
    w.k = k
    w.n_crit = 128                    # every channel: identical rows score identically
    topk_case(w)


def _region_external(values, probs, top_k, seed=0, k_max=None):
    """External scores drawn from a few values over three sequences of 12000-17000 tokens."""
    w = W.batched_joint(batch=3, lo=12000, hi=17000, n_window=128)
    rng = np.random.default_rng(seed)
    vals = np.asarray(values, np.float32)
    acc = vals[rng.choice(len(vals), size=w.acc.shape, p=probs)]
    for b in range(w.batch):
        acc[b, :, w.seq_lens[b]:] = 0.0
    w.acc = acc.astype(np.float32)
    w.top_k = np.asarray(top_k, np.int32)
    return topk_case(w, k_max=k_max)


@pytest.mark.parametrize("top_k", [[3000, 1, 9000], [0, 2500, 20000]])
def test_region_path_all_scores_equal(top_k):
    """One value everywhere: the threshold bin holds every candidate (more than fit in LDS),
    so the first k candidates by index are the answer; k = 0 and k above the candidates too."""
    _region_external([0.5], [1.0], top_k)


def test_region_path_one_bin_many_digits():
    """Three values inside one coarse bin (same sign, exponent and top mantissa bits): a bin
    too large for LDS whose keys differ only in later digits."""
    _region_external([1.0, 1.0000001, 1.0000002], [0.5, 0.3, 0.2], [2000, 7000, 11000], seed=1)


def test_region_path_bin_with_ties_in_lds():
    """Value classes of a few thousand items: the boundary inside a class that fits in LDS."""
    _region_external([1.0, 2.0, 4.0], [0.6, 0.3, 0.1], [2000, 5000, 100], seed=2)


def test_region_path_extreme_exponents():
    """Scores outside the coarse bins' exponent window (clamped into the end bins), zero and
    negative values."""
    _region_external([-1e30, -2.5, 1e-30, 0.0, 7.0, 3e30], [1 / 6] * 6, [4000, 6000, 10], seed=3)


@pytest.mark.parametrize("make", [lambda: W.sparse_crit8(), lambda: W.batched_joint()],
                         ids=["crit8_top4096_128k", "batch16_external"])
def test_full_size(make):
    w = make()
    pairs = [(0, 0), (0, w.hkv - 1)] + ([(w.batch - 1, 3)] if w.batch > 1 else [])
    res = ST.decode_step(w, append=False, pairs=pairs)
    cache = cache_for(w)
    prefill(cache, w)
    km = int(w.top_k.max())
    idx, sc, ch = run_topk(cache, w, km)
    check_topk(w, res, idx, sc, ch, km)
    # every row is ascending, unique, within range and has exactly k_b entries
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        kb = min(int(w.top_k[b]), max(0, n - w.n_window - w.n_sink))
        for g in range(w.hkv):
            r = idx[b, g]
            v = r[r >= 0]
            assert len(v) == kb and np.all(np.diff(v) > 0)
            assert v.min(initial=w.n_sink) >= w.n_sink and v.max(initial=0) < n - w.n_window


# ---------------------------------------------------------------- H2O accumulation

def run_accum(cache, w, logits, stride, lse, sel, k_max):
    acc = dev(w.acc.copy())
    kvc.kvc_accum_scores(cache.desc, w.hq, logits, stride, lse, kvc.MODE[w.mode],
                         dev(sel) if sel is not None else None, k_max, w.n_sink, w.n_window, acc)
    torch.cuda.synchronize()
    return host(acc)


def accum_case(w, append=False, pad=0):
    res = ST.decode_step(w, append=append)
    cache = cache_for(w)
    prefill(cache, w)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    km = int(w.top_k.max()) if w.top_k is not None else 0
    sel = sel_tensor(res, w, km) if km else None
    mode = kvc.MODE[w.mode]
    B, hq = w.batch, w.hq
    stride = (w.n_sink + km + w.n_window if w.mode == "drop" else cache.max_tokens) + pad
    out = torch.empty(B, hq, 128, device="cuda")
    lse = torch.empty(B, hq, device="cuda")
    lg = torch.full((B, hq, stride), float("nan"), device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, hq, mode, km, w.n_sink, w.n_window)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
    kvc.kvc_attend_decode(cache.desc, dev(w.q), hq, w.sm_scale, mode, dev(sel) if sel is not None else None,
                          km, w.n_sink, w.n_window, out, lse, lg, stride, ws, nb)
    acc = run_accum(cache, w, lg, stride, lse, sel, km)
    for (b, g), ref in ((k, res.acc[k[0], k[1]]) for k in res.tokens):
        n = res.caches[(b, g)].n
        assert_close(acc[b, g, :n], ref[:n], f"acc b={b} g={g}")
        assert np.array_equal(acc[b, g, n:], w.acc[b, g, n:]), "tokens past the end are untouched"
        # each step adds exactly G units of probability mass
        assert abs(float(acc[b, g].astype(np.float64).sum() - w.acc[b, g].astype(np.float64).sum())
                   - w.group) < 1e-3


def test_accum_drop_fp16():
    accum_case(W.sparse_crit8(n_ctx=3000, n_planted=40, top_k=200))


def test_accum_drop_sinks_window_int4():
    w = W.single_head_4k(2000)
    w.accumulate = True
    w.acc = np.random.default_rng(2).random((1, 1, w.max_tokens)).astype(np.float32)
    accum_case(w, append=True)


def test_accum_keep_paged():
    accum_case(W.batched_joint(batch=3, lo=500, hi=900, n_window=128))


@pytest.mark.parametrize("n,pad", [(1000, 0), (1001, 0), (1003, 3)])
def test_accum_dense(n, pad):
    """Four tokens a thread with a ragged last quad, and (odd logits stride) one a thread."""
    w = W.int4_dense(n)
    w.accumulate = True
    w.acc = np.random.default_rng(n).random((1, w.hkv, w.max_tokens)).astype(np.float32)
    accum_case(w, pad=pad)
