"""Drop, keep and blocks mode in every cache format that supports them, with the attend
workspace filled with 0xFF bytes before the call (NaN partials, all-ones selection words,
row plans and group lists): its contents on entry are ignored, so o / lse / logits match the
oracle.  Two ragged sequences on 64-token pages; the selection comes from external
(cumulative) scores, per token or per 64-token block."""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_close, cache_for, prefill
from oracle import step as ST
from test_gpu_attend import check_against_oracle, run_attend, sel_tensor
from test_gpu_blocks import block_positions

pytestmark = pytest.mark.gpu

CASES = [("drop", f) for f in ("fp16", "fp8", "int4", "int1")] + \
        [("keep", f) for f in ("int4", "int1")] + \
        [("blocks", f) for f in ("fp16", "fp8", "int4", "int1")]


def _workload(mode, fmt):
    w = W.batched_joint(batch=2, lo=1100, hi=1700, n_window=128, page=64)
    w.fmt, w.mode, w.accumulate = fmt, mode, False
    if mode == "blocks":
        w.granule = "block"
        w.top_k = np.array([4, 7], np.int32)
    return w


@pytest.mark.parametrize("mode,fmt", CASES, ids=[f"{m}-{f}" for m, f in CASES])
def test_stale_workspace(mode, fmt):
    w = _workload(mode, fmt)
    res = ST.decode_step(w, append=False)
    cache = cache_for(w)
    prefill(cache, w)
    k_max = int(w.top_k.max())
    sel = sel_tensor(res, w, k_max)
    if mode != "blocks":
        out, lse, lg, stride = run_attend(cache, w, sel, k_max, fill=255)
        check_against_oracle(w, res, out, lse, lg, k_max, stride)
        return
    # blocks: logits positions [sinks | 64 per selected block | window]
    out, lse, lg, stride = run_attend(cache, w, sel, k_max, fill=255)
    G = w.group
    assert_close(out, res.o, "o")
    assert_close(lse, res.lse, "lse")
    for (b, g), toks in res.tokens.items():
        n = res.caches[(b, g)].n
        pos = block_positions(toks, sel[b, g], n, w.n_sink, w.n_window, k_max)
        rows = lg[b, g * G:(g + 1) * G]
        assert_close(rows[:, pos], res.logits[(b, g)], f"logits b={b} g={g}")
        attended = np.zeros(rows.shape[1], bool)
        attended[pos] = True
        assert np.all(np.isneginf(rows[:, ~attended])), "unattended positions must hold -inf"
