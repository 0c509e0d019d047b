"""kvc_attend_decode_noalloc (the attend call for callers that cannot allocate:
its workspace is the library's static device scratch) against kvc_attend_decode
with a caller workspace, through the C ABI: two calls in a row on one GPU, the
second with a smaller input, each result equal to the workspace call's."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import step as ST

pytestmark = pytest.mark.gpu


def _sel(res, w, k_max):
    sel = np.full((w.batch, w.hkv, k_max), -1, np.int32)
    for (b, g), s in res.sel.items():
        sel[b, g, : len(s)] = s[:k_max]
    return sel


def _both(cache, w, sel=None, k_max=0):
    """(out, lse, logits) of the workspace call and of the no-alloc call."""
    mode = kvc.MODE[w.mode]
    stride = w.n_sink + k_max + w.n_window if w.mode == "drop" else cache.max_tokens
    sel_t = dev(sel) if sel is not None else None
    q = dev(w.q)
    res = []
    for noalloc in (False, True):
        out = torch.full((w.batch, w.hq, 128), float("nan"), device="cuda")
        lse = torch.full((w.batch, w.hq), float("nan"), device="cuda")
        lg = torch.full((w.batch, w.hq, stride), float("nan"), device="cuda")
        if noalloc:
            kvc.kvc_attend_decode_noalloc(cache.desc, q, w.hq, w.sm_scale, mode, sel_t, k_max,
                                          w.n_sink, w.n_window, out, lse, lg, stride)
        else:
            nb = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, w.hq, mode, k_max, w.n_sink,
                                         w.n_window)
            ws = torch.full((max(nb, 16),), 255, dtype=torch.uint8, device="cuda")
            kvc.kvc_attend_decode(cache.desc, q, w.hq, w.sm_scale, mode, sel_t, k_max, w.n_sink,
                                  w.n_window, out, lse, lg, stride, ws, nb)
        torch.cuda.synchronize()
        res.append((host(out), host(lse), host(lg)))
    return res


def _check(ref, got, what):
    """Same kernels, same plan: the scratch call reproduces the workspace call bit for bit
    (logits positions past a sequence's length are written by neither and keep the NaN
    both outputs were filled with)."""
    for a, b, name in zip(ref, got, ("out", "lse", "logits")):
        assert a.shape == b.shape
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: {name} differs"


def test_noalloc_two_calls_second_smaller():
    # call 1: a keep-mode batch on a paged INT4 cache (split partials, selection
    # bitmaps and row plans all in the scratch)
    w1 = W.batched_joint(batch=3, lo=900, hi=1500, n_window=128)
    res1 = ST.decode_step(w1, append=False)
    c1 = cache_for(w1)
    prefill(c1, w1)
    k1 = int(w1.top_k.max())
    ref1, got1 = _both(c1, w1, _sel(res1, w1, k1), k1)
    _check(ref1, got1, "call 1")
    assert_close(got1[0], res1.o, "call 1 vs oracle: o")
    assert_close(got1[1], res1.lse, "call 1 vs oracle: lse")
    # call 2: a smaller dense INT4 cache; the scratch still holds call 1's contents
    w2 = W.int4_dense(700)
    res2 = ST.decode_step(w2, append=False)
    c2 = cache_for(w2)
    prefill(c2, w2)
    ref2, got2 = _both(c2, w2)
    _check(ref2, got2, "call 2")
    assert_close(got2[0], res2.o, "call 2 vs oracle: o")
    assert_close(got2[1], res2.lse, "call 2 vs oracle: lse")
