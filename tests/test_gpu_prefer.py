"""GPU parity of kvc_topk_mass (TailorKV article section 2.1, dense preference
score) against the oracle's top-k probability mass of the same attention rows:
within 1e-3 + 2e-3 |ref| on dense INT4 / 1-bit / fp16 layers, ragged k, planted
ties, k beyond the row and empty rows; the decision P > 0.2 on the two 128K layers."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import select as S
from oracle import step as ST
from test_gpu_attend import run_attend

pytestmark = pytest.mark.gpu


def topk_mass(cache, hq, logits, stride, lse, k, out):
    """kvc_topk_mass with a workspace of the size the library asks for, filled with 0xFF
    (its contents on entry must not matter)."""
    nb = kvc.kvc_workspace_bytes(kvc.OP_TOPK_MASS, cache.desc, hq)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    kvc.kvc_topk_mass(cache.desc, hq, logits, stride, lse, k, out, ws, nb)


def mass_case(w, ks, pairs=None):
    res = ST.decode_step(w, append=False, pairs=pairs)
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, lg, stride = run_attend(cache, w)
    lg_t, lse_t = dev(lg), dev(lse)
    G = w.group
    got = {}
    for k in ks:
        m = torch.full((w.batch, w.hq), float("nan"), device="cuda")
        topk_mass(cache, w.hq, lg_t, stride, lse_t, k, m)
        torch.cuda.synchronize()
        m = host(m)
        got[k] = m
        for (b, g) in res.tokens:
            for j in range(G):
                h = g * G + j
                p = np.exp(res.logits[(b, g)][j] - res.lse[b, h])
                ref = S.topk_mass(p, k)
                assert_close(m[b, h], ref, f"mass k={k} b={b} h={h}")
    return res, got


@pytest.mark.parametrize("fmt", ["int4", "int1", "fp16"])
def test_dense_layers(fmt):
    w = W.int4_dense(3000)
    w.fmt = fmt
    mass_case(w, [0, 1, 17, 128, 2999, 3000, 5000], pairs=[(0, 0), (0, 5)])


def test_planted_ties():
    """Equal logits around the k-th entry: the mass is the same whichever are counted."""
    w = W.int4_dense(1000)
    w.fmt = "fp16"
    w.k[0, 100:300, 2] = w.k[0, 100, 2]       # 200 identical keys in KV head 2
    mass_case(w, [50, 150, 250], pairs=[(0, 2)])


def test_empty_rows():
    w = W.int4_dense(64)
    w.seq_lens = np.array([0], np.int32)
    cache = cache_for(w)
    lg = torch.zeros(1, w.hq, cache.max_tokens, device="cuda")
    lse = torch.zeros(1, w.hq, device="cuda")
    m = torch.full((1, w.hq), float("nan"), device="cuda")
    topk_mass(cache, w.hq, lg, cache.max_tokens, lse, 8, m)
    torch.cuda.synchronize()
    assert np.all(host(m) == 0)


def test_full_size_layers_decision():
    """The 128K 1-bit layer and the planted-key fp16 layer: top-3% mass on a sampled
    KV head's query heads matches the oracle, and so do P (one query row per head,
    averaged) and the quantization-friendly decision at tau = 0.2."""
    k = 3932   # 3% of 131072
    for name, fix in [("llama8b_layer_int1_dense_128k", None),
                      ("llama8b_layer_fp16_crit8_top4096_128k", "dense")]:
        w = W.FULL[name]()
        if fix:
            w.mode, w.score, w.accumulate = "dense", None, False
        res, m = mass_case(w, [k], pairs=[(0, 0)])
        ref = [S.topk_mass(np.exp(res.logits[(0, 0)][j] - res.lse[0, j]), k) for j in range(w.group)]
        p_gpu = S.dense_preference(m[k][0, :w.group]) / w.group
        p_ref = S.dense_preference(ref) / w.group
        assert abs(p_gpu - p_ref) <= 1e-3 + 2e-3 * abs(p_ref), (name, p_gpu, p_ref)
        if abs(p_ref - 0.2) > 1e-2:
            assert S.quantization_friendly(p_gpu) == S.quantization_friendly(p_ref), name


def test_full_size_concentrated_layer_decision():
    """The other branch of the classifier at full size: the 128K fp16 layer with 300 keys per
    KV head turned onto their query head's direction at a large norm, so each row's top 3%
    holds nearly all of its probability (P far below tau: sparsity-friendly); mass, P and
    the decision match the oracle."""
    k = 3932
    w = W.FULL["llama8b_layer_fp16_crit8_top4096_128k"]()
    w.mode, w.score, w.accumulate = "dense", None, False
    rng = np.random.default_rng(21)
    kk = w.k.copy()
    g = 0
    for j, t in enumerate(rng.choice(131072, 300, replace=False)):
        qh = w.q[0, 4 * g + j % 4].astype(np.float64)
        kk[0, t, g] = (qh / np.linalg.norm(qh) * 40.0).astype(np.float16)
    w.k = kk
    res, m = mass_case(w, [k], pairs=[(0, 0)])
    ref = [S.topk_mass(np.exp(res.logits[(0, 0)][j] - res.lse[0, j]), k) for j in range(w.group)]
    p_gpu = S.dense_preference(m[k][0, :w.group]) / w.group
    p_ref = S.dense_preference(ref) / w.group
    assert p_ref < 0.1, p_ref   # the layer really is on the sparsity-friendly side
    assert abs(p_gpu - p_ref) <= 1e-3 + 2e-3 * abs(p_ref), (p_gpu, p_ref)
    assert not S.quantization_friendly(p_gpu) and not S.quantization_friendly(p_ref)


def test_bucket_larger_than_lds():
    """40000 equal logits share one first-level bucket, more keys than the finishing
    kernel stages in LDS: they are re-read from the slices' regions, and the mass is
    k / n."""
    w = W.int4_dense(40000)
    w.fmt = "fp16"
    w.k[0, :, 1] = w.k[0, 0, 1]
    mass_case(w, [1, 3000, 40000], pairs=[(0, 1)])


def test_wider_logits_stride():
    """Rows further apart than the cache capacity (logits_stride > max_tokens)."""
    w = W.int4_dense(700)
    w.fmt = "fp16"
    res = ST.decode_step(w, append=False, pairs=[(0, 4)])
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, lg, stride = run_attend(cache, w)
    wide = np.full((1, w.hq, stride + 40), -1e30, np.float32)
    wide[:, :, :stride] = lg
    m = torch.full((1, w.hq), float("nan"), device="cuda")
    topk_mass(cache, w.hq, dev(wide), stride + 40, dev(lse), 33, m)
    torch.cuda.synchronize()
    for j in range(w.group):
        h = 4 * w.group + j
        p = np.exp(res.logits[(0, 4)][j] - res.lse[0, h])
        assert_close(host(m)[0, h], S.topk_mass(p, 33), f"h={h}")
