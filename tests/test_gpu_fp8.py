"""GPU parity of the FP8 (E4M3) warm tier (meeting-LLM article section 6.2; KV
compression survey section 2): codes written by kvc_quantize_append bit for bit
against the oracle on every finite fp16 value, scores and Top-K on FP8 caches bit
for bit, and attention (dense, drop, blocks; contiguous and paged) within
1e-3 + 2e-3 |ref|, including the 128K layer."""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_sparse_kvc_amd import KvcCache, kvc
from gpu_util import assert_close, cache_for, dev, host, prefill
from oracle import quant as Q
from oracle import step as ST
from test_gpu_attend import check_against_oracle, run_attend, sel_tensor
from test_gpu_blocks import block_case
from test_gpu_topk import topk_case

pytestmark = pytest.mark.gpu


def test_codes_every_fp16_value():
    """Append rows holding all 63488 finite fp16 values (K and V) and compare the codes,
    the channel-major copy (decoded values) and max |K|."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    n = x.size // 128                          # 496 tokens
    rows = x[: n * 128].reshape(n, 128)
    k = np.ascontiguousarray(rows[None, :, None, :])          # [1, n, 1, 128]
    v = np.ascontiguousarray(rows[::-1][None, :, None, :])
    cap = ((n + 63) // 64) * 64
    cache = KvcCache("fp8", 1, 1, cap, kT=True)
    cache.append(dev(k), dev(v), dev(np.array([n], np.int32)))
    torch.cuda.synchronize()
    kc = host(cache.k_codes).reshape(cap, 128)[:n]
    vc = host(cache.v_codes).reshape(cap, 128)[:n]
    assert np.array_equal(kc, Q.encode_fp8(k[0, :, 0]))
    assert np.array_equal(vc, Q.encode_fp8(v[0, :, 0]))
    kt = host(cache.kT)[0, 0, :, :n].T.astype(np.float64)
    assert np.array_equal(kt, Q.decode_fp8(kc))
    assert int(host(cache.seq_lens)[0]) == n


@pytest.mark.parametrize("n", [1, 63, 777, 4097])
def test_dense(n):
    w = W.fp8_dense(n_ctx=n)
    res = ST.decode_step(w, append=True, pairs=[(0, 0), (0, 3), (0, 7)])
    cache = cache_for(w)
    prefill(cache, w)
    cache.append(dev(w.k_new), dev(w.v_new))
    out, lse, lg, stride = run_attend(cache, w)
    G = w.group
    for (b, g), toks in res.tokens.items():
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")
        assert_close(lg[b, sl][:, toks], res.logits[(b, g)], f"logits g={g}")


def test_dense_paged():
    w = W.fp8_dense(n_ctx=3000)
    page = 16
    per = w.max_tokens // page
    w.page_size, w.num_pages = page, per
    w.block_table = np.random.default_rng(8).permutation(per).astype(np.int32)[None]
    res = ST.decode_step(w, append=False, pairs=[(0, 2), (0, 5)])
    cache = cache_for(w)
    prefill(cache, w)
    out, lse, lg, stride = run_attend(cache, w)
    G = w.group
    for (b, g) in res.tokens:
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")


@pytest.mark.parametrize("kT", [False, True])
def test_critical_topk_drop(kT):
    w = W.sparse_crit8(n_ctx=3000, n_planted=40, top_k=200)
    w.fmt, w.kT = "fp8", kT
    res, cache, idx = topk_case(w)
    km = int(w.top_k.max())
    sel = sel_tensor(res, w, km)
    out, lse, lg, stride = run_attend(cache, w, sel, km)
    check_against_oracle(w, res, out, lse, lg, km, stride)


def test_exact_topk_sinks_window():
    w = W.single_head_4k(2000)
    w.fmt = "fp8"
    res, cache, idx = topk_case(w, append=True)
    km = int(w.top_k.max())
    out, lse, lg, stride = run_attend(cache, w, sel_tensor(res, w, km), km)
    check_against_oracle(w, res, out, lse, lg, km, stride)


def test_blocks():
    w = W.sparse_blocks(n_ctx=4097, fmt="fp8", top_blocks=7)
    w.n_sink, w.n_window = 4, 100
    block_case(w, append=True, pairs=[(0, 1), (0, 6)])


def test_keep_is_unsupported():
    w = W.fp8_dense(n_ctx=100)
    cache = cache_for(w)
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, cache.desc, w.hq, kvc.MODE["keep"], 4, 0, 0) == 0


def test_full_size_dense():
    """The 128K FP8 layer in the benchmark's launch configuration, sampled pairs."""
    w = W.FULL["llama8b_layer_fp8_dense_128k"]()
    res = ST.decode_step(w, append=True, pairs=[(0, 0), (0, 6)])
    cache = cache_for(w)
    prefill(cache, w)
    cache.append(dev(w.k_new), dev(w.v_new))
    out, lse, _, _ = run_attend(cache, w, logits=False)
    G = w.group
    for (b, g) in res.tokens:
        sl = slice(g * G, (g + 1) * G)
        assert_close(out[b, sl], res.o[b, sl], f"o g={g}")
        assert_close(lse[b, sl], res.lse[b, sl], f"lse g={g}")


def test_ragged_paged_appends():
    """Three sequences on a shared, shuffled 16-token page pool appended in ragged
    steps: every slot's codes equal the oracle's cast of the appended value."""
    rng = np.random.default_rng(21)
    B, hkv, page, cap = 3, 2, 16, 256
    per = cap // page
    table = torch.from_numpy(rng.permutation(B * per).astype(np.int32).reshape(B, per))
    cache = KvcCache("fp8", B, hkv, cap, page_size=page, block_table=table, num_pages=B * per)
    rows = [np.zeros((0, hkv, 128), np.float16) for _ in range(B)]
    for step in range(4):
        n_new = rng.integers(0, 70, size=B).astype(np.int32)
        m = int(n_new.max())
        k = (rng.normal(size=(B, max(m, 1), hkv, 128)) * 30).astype(np.float16)
        v = rng.normal(size=(B, max(m, 1), hkv, 128)).astype(np.float16)
        cache.append(dev(k), dev(v), dev(n_new))
        for b in range(B):
            rows[b] = np.concatenate([rows[b], k[b, : n_new[b]]])
    torch.cuda.synchronize()
    lens = host(cache.seq_lens)
    kc = host(cache.k_codes).reshape(-1, 128)
    tab = table.numpy()
    for b in range(B):
        assert lens[b] == rows[b].shape[0]
        for t in range(int(lens[b])):
            phys = tab[b, t // page]
            for g in range(hkv):
                slot = (phys * hkv + g) * page + t % page
                assert np.array_equal(kc[slot], Q.encode_fp8(rows[b][t, g])), (b, t, g)
