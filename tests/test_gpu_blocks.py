"""GPU parity of block-granular selection and block-sparse attention (meeting-LLM
article, section 8.1): kvc_score_topk with KVC_SCORE_BLOCKS (block means and block
ids bit for bit), kvc_attend_decode in KVC_ATTEND_BLOCKS mode and the H2O update
over its positions (within 1e-3 + 2e-3 |ref|), on fp16 / INT4 / 1-bit caches with
and without sinks and a window, ragged tails, and the 128K workloads."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import select as S
from oracle import step as ST
from test_gpu_attend import sel_tensor
from test_gpu_topk import run_accum

pytestmark = pytest.mark.gpu


def run_block_topk(cache, w, k_max):
    B, hkv = w.batch, w.hkv
    idx = torch.full((B, hkv, max(k_max, 1)), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, hkv, cache.max_tokens), float("nan"), dtype=torch.float64, device="cuda")
    ch = torch.full((B, hkv, w.n_crit), -7, dtype=torch.int32, device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, cache.desc, w.hq)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ext = dev(w.acc) if w.score == "external" else None
    kvc.kvc_score_topk(cache.desc, dev(w.q), w.hq, kvc.SCORE[w.score] | kvc.SCORE_BLOCKS, w.n_crit,
                       ext, w.n_sink, w.n_window, dev(w.top_k.astype(np.int32)), k_max, idx, sc,
                       ch, ws, nb)
    torch.cuda.synchronize()
    return host(idx)[:, :, :k_max], host(sc)


def block_positions(toks, sel, n, n_sink, n_window, k_max):
    """Logits position of each attended token in blocks mode (header convention)."""
    w0 = max(n - n_window, min(n_sink, n))
    where = {int(j): i for i, j in enumerate(sel) if j >= 0}
    pos = []
    for t in toks:
        t = int(t)
        if t < n_sink:
            pos.append(t)
        elif t >= w0:
            pos.append(n_sink + 64 * k_max + t - w0)
        else:
            pos.append(n_sink + 64 * where[t // 64] + t % 64)
    return np.array(pos, np.int64)


def run_block_attend(cache, w, sel, k_max):
    mode = kvc.MODE["blocks"]
    B, hq = w.batch, w.hq
    stride = w.n_sink + 64 * k_max + w.n_window
    out = torch.full((B, hq, 128), float("nan"), device="cuda")
    lse = torch.full((B, hq), float("nan"), device="cuda")
    lg = torch.full((B, hq, stride), float("nan"), device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, hq, mode, k_max, w.n_sink, w.n_window)
    assert nb > 0
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    kvc.kvc_attend_decode(cache.desc, dev(w.q), hq, w.sm_scale, mode, dev(sel), k_max, w.n_sink,
                          w.n_window, out, lse, lg, stride, ws, nb)
    torch.cuda.synchronize()
    return host(out), host(lse), host(lg), stride, lse


def block_case(w, append=False, pairs=None, k_max=None, accumulate=True):
    res = ST.decode_step(w, append=append, pairs=pairs)
    cache = cache_for(w)
    prefill(cache, w)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    km = int(w.top_k.max()) if k_max is None else k_max
    idx, sc = run_block_topk(cache, w, km)
    for (b, g), ref_sel in res.sel.items():
        n = res.caches[(b, g)].n
        lo, hi = S.block_range(n, w.n_sink, w.n_window)
        where = f"b={b} g={g}"
        if hi > lo:
            got = sc[b, g, lo:hi]
            ref = res.scores[(b, g)][lo:hi]
            assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), "block means " + where
        want = np.full(km, -1, np.int64)
        want[: len(ref_sel)] = ref_sel[:km]
        assert np.array_equal(idx[b, g], want), f"blocks {where}: {idx[b, g][:12]} vs {want[:12]}"
    # the GPU's own selection feeds the attention (equal to the oracle's, checked above)
    sel = np.ascontiguousarray(idx.astype(np.int32))
    out, lse, lg, stride, lse_t = run_block_attend(cache, w, sel, km)
    G = w.group
    for (b, g), toks in res.tokens.items():
        n = res.caches[(b, g)].n
        assert_close(out[b, g * G:(g + 1) * G], res.o[b, g * G:(g + 1) * G], f"o b={b} g={g}")
        assert_close(lse[b, g * G:(g + 1) * G], res.lse[b, g * G:(g + 1) * G], f"lse b={b} g={g}")
        pos = block_positions(toks, sel[b, g], n, w.n_sink, w.n_window, km)
        rows = lg[b, g * G:(g + 1) * G]
        assert_close(rows[:, pos], res.logits[(b, g)], f"logits b={b} g={g}")
        attended = np.zeros(stride, bool)
        attended[pos] = True
        assert np.all(np.isneginf(rows[:, ~attended])), "unattended positions must hold -inf"
    if accumulate and w.accumulate:
        lg_t = dev(lg)
        acc = run_accum(cache, w, lg_t, stride, lse_t, sel, km)
        for (b, g) in res.tokens:
            n = res.caches[(b, g)].n
            assert_close(acc[b, g, :n], res.acc[b, g, :n], f"acc b={b} g={g}")
    return res, cache


@pytest.mark.parametrize("fmt", ["fp16", "int4", "int1"])
@pytest.mark.parametrize("n,top", [(3000, 5), (4097, 20), (700, 40)])
def test_blocks_critical(fmt, n, top):
    w = W.sparse_blocks(n_ctx=n, fmt=fmt, top_blocks=top)
    block_case(w, pairs=[(0, 0), (0, 3), (0, 7)])


@pytest.mark.parametrize("fmt", ["fp16", "int4"])
def test_blocks_sinks_window_and_append(fmt):
    w = W.sparse_blocks(n_ctx=5000, fmt=fmt, top_blocks=9)
    w.n_sink, w.n_window = 4, 300
    block_case(w, append=True, pairs=[(0, 1), (0, 6)])


def test_blocks_exact_and_external_scores():
    w = W.sparse_blocks(n_ctx=2500, fmt="int4", top_blocks=6)
    w.score = "exact"
    block_case(w, pairs=[(0, 2)])
    w2 = W.sparse_blocks(n_ctx=2500, fmt="int4", top_blocks=6)
    w2.score = "external"
    w2.acc = np.random.default_rng(5).lognormal(0, 1.5, size=w2.acc.shape).astype(np.float32)
    w2.accumulate = False
    block_case(w2, pairs=[(0, 4)])


def test_blocks_long_range_histogram():
    """More than 8192 candidate blocks (one pair of 528K tokens, external scores with
    planted equal block means): the block keys are counted into histogram slots by
    block-key workgroups that each take several rounds of blocks, and the long-range path
    selects; block means and ids equal the oracle's bit for bit."""
    from decode_attention_sparse_kvc_amd import KvcCache
    n = 8300 * 64 + 37
    cap = -(-(n + 1) // 64) * 64
    cache = KvcCache("fp16", 1, 1, cap)
    cache.seq_lens.fill_(n)
    rng = np.random.default_rng(61)
    ext = rng.lognormal(0.0, 1.5, size=(1, 1, cap)).astype(np.float32)
    ext[..., n:] = 0.0
    for blk in rng.choice(8000, 40, replace=False):          # 40 blocks with one equal mean
        ext[0, 0, 64 * (blk + 1): 64 * (blk + 2)] = 5.0
    n_sink, n_window, k, k_max = 4, 64, 600, 700
    idx = torch.full((1, 1, k_max), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((1, 1, cap), float("nan"), dtype=torch.float64, device="cuda")
    nb = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, cache.desc, 1)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    q = torch.zeros((1, 1, 128), dtype=torch.float16, device="cuda")
    kvc.kvc_score_topk(cache.desc, q, 1, kvc.SCORE["external"] | kvc.SCORE_BLOCKS, 8, dev(ext),
                       n_sink, n_window, dev(np.array([k], np.int32)), k_max, idx, sc, None, ws, nb)
    torch.cuda.synchronize()
    r = ext[0, 0].astype(np.float64)
    lo, hi = S.block_range(n, n_sink, n_window)
    assert hi - lo > 8192
    bs = S.block_scores(r, lo, hi)
    got = host(sc)[0, 0, lo:hi]
    assert np.array_equal(got.view(np.uint64), bs[lo:hi].view(np.uint64)), "block means"
    want = S.topk_indices(bs, lo, hi, k, k_max)
    assert np.array_equal(host(idx)[0, 0], want), (host(idx)[0, 0][:12], want[:12])


def test_blocks_more_than_candidates_and_empty():
    w = W.sparse_blocks(n_ctx=1000, fmt="int4", top_blocks=50)   # 15 candidates, k_max 50
    block_case(w, pairs=[(0, 0)])
    w2 = W.sparse_blocks(n_ctx=100, fmt="int1", top_blocks=3)    # one candidate block
    w2.n_window = 40
    block_case(w2, pairs=[(0, 5)])


@pytest.mark.parametrize("fmt", ["fp16", "int4"])
def test_blocks_full_size(fmt):
    """The 128K block workloads in the benchmark's configuration; every pair's block
    selection and attention against the oracle on two sampled pairs."""
    w = W.FULL[f"llama8b_layer_{fmt}_crit8_block61_128k"]()
    block_case(w, pairs=[(0, 0), (0, 5)])


def test_blocks_paged_fp16():
    """Blocks mode on a paged fp16 store (plan kernel, page table) with sinks and window."""
    w = W.sparse_blocks(n_ctx=3000, fmt="fp16", top_blocks=6)
    w.kT = False
    w.n_sink, w.n_window = 4, 70
    page = 16
    per = w.max_tokens // page
    w.page_size, w.num_pages = page, per
    w.block_table = np.random.default_rng(13).permutation(per).astype(np.int32)[None]
    block_case(w, pairs=[(0, 3)])


def test_blocks_no_selection():
    """k_max = 0: only the sinks and the window are attended (quantized and fp16)."""
    for fmt in ["int4", "fp16"]:
        w = W.sparse_blocks(n_ctx=2000, fmt=fmt, top_blocks=0)
        w.n_sink, w.n_window = 4, 200
        w.score = None
        res = ST.decode_step(w, append=False, pairs=[(0, 1)])
        cache = cache_for(w)
        prefill(cache, w)
        sel = np.zeros((1, w.hkv, 1), np.int32)
        out, lse, lg, stride, _ = run_block_attend(cache, w, sel, 0)
        G = w.group
        assert_close(out[0, G:2 * G], res.o[0, G:2 * G], f"o {fmt}")
        assert_close(lse[0, G:2 * G], res.lse[0, G:2 * G], f"lse {fmt}")
