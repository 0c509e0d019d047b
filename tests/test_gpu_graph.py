"""HIP graph replay of whole decode steps (append, score + Top-K, attend, H2O
accumulation) matches the same calls launched one by one: the graph is
replayed several times, with eager calls and synchronizations between the
replays, and every replay is compared bit for bit with the eager step."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import cache_for, dev, host, prefill
from test_gpu_attend import paged

pytestmark = pytest.mark.gpu

STEPS = 4


class Path:
    """One cache and its own buffers for the step's calls."""

    def __init__(self, w):
        self.w = w
        self.cache = cache_for(w)
        prefill(self.cache, w)
        B, hq, hkv = w.batch, w.hq, w.hkv
        self.k_max = int(w.top_k.max())
        self.mode = kvc.MODE[w.mode]
        self.stride = self.cache.max_tokens
        self.q, self.k_new, self.v_new = dev(w.q), dev(w.k_new), dev(w.v_new)
        self.kps = dev(w.top_k.astype(np.int32))
        self.acc = torch.zeros(B, hkv, self.cache.max_tokens, device="cuda")
        self.acc[:, :, : w.acc.shape[2]] = dev(w.acc[:, :, : self.cache.max_tokens])
        self.sel = torch.full((B, hkv, self.k_max), -1, dtype=torch.int32, device="cuda")
        self.out = torch.zeros(B, hq, 128, device="cuda")
        self.lse = torch.zeros(B, hq, device="cuda")
        self.lg = torch.zeros(B, hq, self.stride, device="cuda")
        self.tk_nb = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, self.cache.desc, hq)
        self.tk_ws = torch.zeros(self.tk_nb, dtype=torch.uint8, device="cuda")
        self.nb = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, self.cache.desc, hq, self.mode, self.k_max,
                                          w.n_sink, w.n_window)
        self.ws = torch.zeros(self.nb, dtype=torch.uint8, device="cuda")

    def step(self, stream):
        w, c = self.w, self.cache
        kvc.kvc_quantize_append(c.desc, self.k_new, self.v_new, None, 1, None, stream)
        kvc.kvc_score_topk(c.desc, self.q, w.hq, kvc.SCORE[w.score], w.n_crit, self.acc, w.n_sink,
                           w.n_window, self.kps, self.k_max, self.sel, None, None, self.tk_ws,
                           self.tk_nb, stream)
        kvc.kvc_attend_decode(c.desc, self.q, w.hq, w.sm_scale, self.mode, self.sel, self.k_max,
                              w.n_sink, w.n_window, self.out, self.lse, self.lg, self.stride,
                              self.ws, self.nb, stream)
        kvc.kvc_accum_scores(c.desc, w.hq, self.lg, self.stride, self.lse, self.mode, self.sel,
                             self.k_max, w.n_sink, w.n_window, self.acc, stream)

    def snapshot(self):
        return {k: host(getattr(self, k)).copy() for k in ("sel", "out", "lse", "acc")}


def test_graph_replay_matches_eager():
    w = W.batched_joint(batch=3, lo=500, hi=900, n_window=128)
    paged(w, 16, room=STEPS + 2)
    eager, graphed = Path(w), Path(w)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    for i in range(STEPS):
        eager.step(stream)
        torch.cuda.synchronize()
        want = eager.snapshot()
        g.replay()
        torch.cuda.synchronize()
        got = graphed.snapshot()
        for k in want:
            assert np.array_equal(got[k], want[k], equal_nan=True), f"replay {i}: {k} differs"
        assert (host(graphed.cache.seq_lens) == w.seq_lens + i + 1).all()
