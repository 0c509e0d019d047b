"""GPU parity of kvc_attend_decode against the oracle (o, lse, logits within
1e-3 + 2e-3 |ref|): dense INT4/INT1/fp16 with ragged tails, drop mode over
gathered tokens, keep mode over a paged INT4 cache with an fp16 keep set,
edge cases, and the full-size 128K INT4 / 1-bit layers in the benchmark's
launch configuration."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import select as S
from oracle import step as ST

pytestmark = pytest.mark.gpu


def sel_tensor(res, w, k_max):
    sel = np.full((w.batch, w.hkv, k_max), -1, np.int32)
    for (b, g), s in res.sel.items():
        sel[b, g, : len(s)] = s[:k_max]
    return sel


def run_attend(cache, w, sel=None, k_max=0, logits=True, workgroups=0, fill=0):
    """kvc_attend_decode on w (workspace bytes preset to `fill`); host out, lse, logits, stride."""
    mode = kvc.MODE[w.mode]
    B, hq = w.batch, w.hq
    out = torch.full((B, hq, 128), float("nan"), device="cuda")
    lse = torch.full((B, hq), float("nan"), device="cuda")
    stride = (w.n_sink + k_max + w.n_window if w.mode == "drop"
              else w.n_sink + 64 * k_max + w.n_window if w.mode == "blocks" else cache.max_tokens)
    lg = torch.full((B, hq, stride), float("nan"), device="cuda") if logits else None
    nbytes = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, hq, mode, k_max, w.n_sink, w.n_window,
                                     workgroups)
    ws = torch.full((max(nbytes, 16),), fill, dtype=torch.uint8, device="cuda")
    sel_t = dev(sel) if sel is not None else None
    kvc.kvc_attend_decode(cache.desc, dev(w.q), hq, w.sm_scale, mode, sel_t, k_max, w.n_sink,
                          w.n_window, out, lse, lg, stride, ws, nbytes, workgroups=workgroups)
    torch.cuda.synchronize()
    return host(out), host(lse), (host(lg) if logits else None), stride


def drop_positions(toks, sel, n, n_sink, n_window, k_max):
    """Logits position of each attended token in drop mode (header convention)."""
    w0 = max(n - n_window, min(n_sink, n))
    where = {int(t): i for i, t in enumerate(sel) if t >= 0}
    pos = []
    for t in toks:
        t = int(t)
        if t < n_sink:
            pos.append(t)
        elif t >= w0:
            pos.append(n_sink + k_max + t - w0)
        else:
            pos.append(n_sink + where[t])
    return np.array(pos, np.int64)


def check_against_oracle(w, res, out, lse, lg, k_max=0, stride=None):
    assert_close(out, res.o, "o")
    assert_close(lse, res.lse, "lse")
    if lg is None:
        return
    G = w.group
    for (b, g), toks in res.tokens.items():
        ref = res.logits[(b, g)]                     # [G, T]
        n = res.caches[(b, g)].n
        if w.mode == "drop":
            pos = drop_positions(toks, res.sel.get((b, g), []), n, w.n_sink, w.n_window, k_max)
            got = lg[b, g * G:(g + 1) * G][:, pos]
            attended = np.zeros(stride, bool)
            attended[pos] = True
            rest = lg[b, g * G:(g + 1) * G][:, ~attended]
            assert np.all(np.isneginf(rest)), "unattended drop positions must hold -inf"
        else:
            got = lg[b, g * G:(g + 1) * G][:, toks]
        assert_close(got, ref, f"logits b={b} g={g}")


def oracle_and_cache(w, append=False):
    res = ST.decode_step(w, append=append)
    cache = cache_for(w)
    prefill(cache, w)
    torch.cuda.synchronize()
    return res, cache


@pytest.mark.parametrize("fmt,n", [("int4", 1000), ("int4", 1024), ("int1", 1000), ("int1", 2048 + 63),
                                   ("fp16", 777)])
def test_dense(fmt, n):
    if fmt == "fp16":
        w = W.int4_dense(n)
        w.fmt = "fp16"
    else:
        w = W.int4_dense(n) if fmt == "int4" else W.int1_dense(n)
    res, cache = oracle_and_cache(w)
    out, lse, lg, stride = run_attend(cache, w)
    check_against_oracle(w, res, out, lse, lg)


def paged(w, page, seed=0, room=1):
    """Move w onto a paged cache: capacity (longest sequence + room) rounded up to
    lcm(page, 64), pages shuffled."""
    unit = int(np.lcm(page, 64))
    cap = -(-(int(w.seq_lens.max()) + room) // unit) * unit
    per = cap // page
    perm = np.random.default_rng(seed).permutation(w.batch * per).astype(np.int32)
    w.page_size, w.block_table = page, perm.reshape(w.batch, per)
    w.num_pages, w.max_tokens = w.batch * per, cap
    return w


@pytest.mark.parametrize("fmt,page", [("int4", 16), ("int4", 48), ("int4", 64), ("int4", 192),
                                      ("int1", 64), ("int1", 192), ("fp16", 48)])
def test_dense_paged(fmt, page):
    """Page lengths that split a 64-token group (16, 48) take one page lookup per tile."""
    w = W.int1_dense(1500) if fmt == "int1" else W.int4_dense(1500)
    w.fmt = fmt
    paged(w, page)
    res, cache = oracle_and_cache(w)
    out, lse, lg, _ = run_attend(cache, w)
    check_against_oracle(w, res, out, lse, lg)


def test_workspace_reuse():
    """One workspace (holding stale partials of earlier calls) serves call after call, also
    when the split count changes between calls; repeated calls agree bit for bit."""
    w = W.int4_dense(3000)
    res, cache = oracle_and_cache(w)
    mode = kvc.MODE[w.mode]
    sizes = {}
    for t in [512, 3, 64]:
        sizes[t] = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, w.hq, mode, 0, 0, 0, t)
    ws = torch.full((max(sizes.values()),), 255, dtype=torch.uint8, device="cuda")   # NaN bytes
    outs = []
    for t in [512, 3, 512, 64, 3]:
        out = torch.full((w.batch, w.hq, 128), float("nan"), device="cuda")
        lse = torch.full((w.batch, w.hq), float("nan"), device="cuda")
        kvc.kvc_attend_decode(cache.desc, dev(w.q), w.hq, w.sm_scale, mode, None, 0, 0, 0,
                              out, lse, None, 0, ws, ws.numel(), workgroups=t)
        torch.cuda.synchronize()
        check_against_oracle(w, res, host(out), host(lse), None)
        outs.append((t, host(out), host(lse)))
    for t, o, l in outs:
        same = [o2 for t2, o2, _ in outs if t2 == t]
        assert all(np.array_equal(o, o2) for o2 in same), f"target {t}: repeated calls differ"


@pytest.mark.parametrize("n", [0, 1, 5, 63, 64, 65])
@pytest.mark.parametrize("fmt", ["int4", "int1", "fp16"])
def test_short_and_empty(fmt, n):
    w = W.int4_dense(max(n, 1))
    w.fmt = fmt
    w.seq_lens = np.array([n], np.int32)
    res, cache = oracle_and_cache(w)
    out, lse, lg, _ = run_attend(cache, w)
    if n == 0:
        assert np.all(out == 0) and np.all(np.isneginf(lse))
    else:
        check_against_oracle(w, res, out, lse, lg)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_group_sizes(G):
    w = W.int4_dense(700)
    w.hkv = 32 // G if G < 8 else 4
    w.hq = w.hkv * G
    rng = np.random.default_rng(5)
    w.k = rng.standard_normal((1, 700, w.hkv, 128), dtype=np.float32).astype(np.float16)
    w.v = rng.standard_normal((1, 700, w.hkv, 128), dtype=np.float32).astype(np.float16)
    w.q = rng.standard_normal((1, w.hq, 128), dtype=np.float32).astype(np.float16)
    res, cache = oracle_and_cache(w)
    out, lse, lg, _ = run_attend(cache, w)
    check_against_oracle(w, res, out, lse, lg)


@pytest.mark.parametrize("make", [lambda: W.single_head_4k(1000), lambda: W.single_head_4k(4096)],
                         ids=["n1000", "n4096"])
def test_drop_int4_exact_topk(make):
    """Single head, sinks + exact Top-K + window over the INT4 cache (sel from the oracle)."""
    w = make()
    res, cache = oracle_and_cache(w)
    k_max = int(w.top_k[0])
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg, k_max, stride)


@pytest.mark.parametrize("n_sink,n_window", [(0, 0), (4, 64), (3, 40)])
def test_drop_fp16_gather(n_sink, n_window):
    w = W.sparse_crit8(n_ctx=3000, n_planted=40, top_k=200)
    w.n_sink, w.n_window = n_sink, n_window
    res, cache = oracle_and_cache(w)
    k_max = 256          # wider than top_k: -1 padding positions
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg, k_max, stride)


@pytest.mark.parametrize("fmt", ["fp16", "fp8"])
def test_drop_paged_rows(fmt):
    """Drop mode on a paged fp16 / FP8 row store (positions planned by the plan kernel,
    rows found through the page table) against the contiguous case's inline planning."""
    w = W.sparse_crit8(n_ctx=3000, n_planted=40, top_k=200)
    w.fmt, w.kT = fmt, False
    w.n_sink, w.n_window = 4, 100
    page = 16
    per = w.max_tokens // page
    w.page_size, w.num_pages = page, per
    w.block_table = np.random.default_rng(12).permutation(per).astype(np.int32)[None]
    res, cache = oracle_and_cache(w)
    k_max = 256
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg, k_max, stride)


def test_drop_int1_and_out_of_range_entries():
    """Drop mode on a 1-bit cache; sel entries inside the sink/window ranges are ignored."""
    w = W.int1_dense(900)
    w.mode, w.n_sink, w.n_window = "drop", 4, 100
    rng = np.random.default_rng(9)
    picks = np.sort(rng.choice(np.arange(4, 800), 50, replace=False))
    sel = np.full((1, w.hkv, 64), -1, np.int32)
    sel[0, :, :50] = picks
    sel[0, :, 50] = 850          # inside the window: ignored
    sel[0, :, 51] = 860
    res = ST.StepResult({}, {}, {}, {}, {}, {}, np.zeros((1, 32, 128)), np.zeros((1, 32)), None)
    for g in range(w.hkv):
        hc = ST.build_head_cache(w.k[0, :900, g], w.v[0, :900, g], "int1")
        keys, vals = ST.token_rows(hc)
        toks = S.attended_tokens("drop", 900, 4, 100, sel[0, g])
        from oracle import attend as A
        o, l, lg = A.attend_group(w.q[0, 4 * g:4 * g + 4], keys[toks], vals[toks], w.sm_scale)
        res.o[0, 4 * g:4 * g + 4], res.lse[0, 4 * g:4 * g + 4] = o, l
        res.tokens[(0, g)], res.logits[(0, g)], res.caches[(0, g)] = toks, lg, hc
        res.sel[(0, g)] = sel[0, g]
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, lg, stride = run_attend(cache, w, sel, 64)
    check_against_oracle(w, res, out, lse, lg, 64, stride)


@pytest.mark.parametrize("append", [False, True])
def test_keep_paged_int4(append):
    """Joint tiers: keep set (sinks + top cumulative-score tokens + window) in fp16, rest INT4."""
    w = W.batched_joint(batch=3, lo=500, hi=900, n_window=128)
    res, cache = oracle_and_cache(w, append=append)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    k_max = int(w.top_k.max())
    out, lse, lg, _ = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg)


@pytest.mark.parametrize("append", [False, True])
def test_keep_paged_int1(append):
    """Joint tiers on a 1-bit cache with 64-token pages: keep set in fp16, rest 1-bit codes."""
    w = W.batched_joint(batch=3, lo=500, hi=900, n_window=128, page=64)
    w.fmt = "int1"
    res, cache = oracle_and_cache(w, append=append)
    if append:
        cache.append(dev(w.k_new), dev(w.v_new))
    k_max = int(w.top_k.max())
    out, lse, lg, _ = run_attend(cache, w, sel_tensor(res, w, k_max), k_max)
    check_against_oracle(w, res, out, lse, lg)


@pytest.mark.parametrize("target", [1, 64, 4096])
def test_split_count_invariance(target):
    """The result does not depend on how the context is split across workgroups."""
    w = W.int4_dense(5000)
    res, cache = oracle_and_cache(w)
    out, lse, lg, _ = run_attend(cache, w, workgroups=target)
    check_against_oracle(w, res, out, lse, lg)


@pytest.mark.parametrize("make", [lambda: W.int4_dense(131072), lambda: W.int1_dense(131072)],
                         ids=["int4_128k", "int1_128k"])
def test_full_size_dense(make):
    """Benchmark workload and launch configuration; oracle on two KV heads (8 query heads)."""
    w = make()
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, lg, _ = run_attend(cache, w, logits=False)
    res = ST.decode_step(w, append=False, pairs=[(0, 0), (0, 5)])
    for g in (0, 5):
        assert_close(out[0, 4 * g:4 * g + 4], res.o[0, 4 * g:4 * g + 4], f"o g={g}")
        assert_close(lse[0, 4 * g:4 * g + 4], res.lse[0, 4 * g:4 * g + 4], f"lse g={g}")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("make,pairs", [
    (lambda: W.batched_joint(), [(0, 0), (7, 3), (15, 7)]),
    (lambda: W.sparse_crit8(), [(0, 0), (0, 6)]),
], ids=["batch16_keep", "crit8_drop_128k"])
def test_full_size_sparse(make, pairs):
    """The benchmark's keep / drop workloads at full size: the GPU Top-K feeds the GPU
    attention and the H2O update (as in a step); on sampled pairs the selection must equal
    the oracle's and o / lse / logits / cumulative scores must match it."""
    from test_gpu_topk import run_topk
    w = make()
    res = ST.decode_step(w, append=False, pairs=pairs)
    cache = cache_for(w)
    prefill(cache, w)
    k_max = int(w.top_k.max())
    idx, _, _ = run_topk(cache, w, k_max, scores=False)
    for (b, g), ref_sel in res.sel.items():
        want = np.full(k_max, -1, np.int64)
        want[: len(ref_sel)] = ref_sel[:k_max]
        assert np.array_equal(idx[b, g], want), f"selection b={b} g={g}"
    out, lse, lg, stride = run_attend(cache, w, idx.astype(np.int32), k_max)
    G = w.group
    for (b, g) in pairs:
        hs = slice(g * G, (g + 1) * G)
        assert_close(out[b, hs], res.o[b, hs], f"o b={b} g={g}")
        assert_close(lse[b, hs], res.lse[b, hs], f"lse b={b} g={g}")
    # logits of the sampled pairs (o / lse were compared above; the rest of res is unsampled)
    sampled = ST.StepResult(res.caches, res.channels, res.scores, res.sel, res.tokens, res.logits,
                            out, lse, None)
    check_against_oracle(w, sampled, out, lse, lg, k_max, stride)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    # the H2O update of the step, on the sampled pairs
    from test_gpu_topk import run_accum
    acc = run_accum(cache, w, dev(lg), stride, dev(lse), np.ascontiguousarray(idx.astype(np.int32)),
                    k_max)
    for (b, g) in pairs:
        n = res.caches[(b, g)].n
        assert_close(acc[b, g, :n], res.acc[b, g, :n], f"acc b={b} g={g}")
        assert np.array_equal(acc[b, g, n:], w.acc[b, g, n:]), "tokens past the end are untouched"
