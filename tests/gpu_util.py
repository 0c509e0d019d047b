"""Helpers for the GPU parity tests: caches from workloads, transfers, tolerance."""
from __future__ import annotations

import numpy as np
import torch

from decode_attention_sparse_kvc_amd import KvcCache

RTOL, ATOL = 2e-3, 1e-3      # elementwise |gpu - ref| <= ATOL + RTOL * |ref|


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def cache_for(w, max_tokens=None) -> KvcCache:
    table = torch.from_numpy(w.block_table) if w.block_table is not None else None
    oc = torch.from_numpy(w.outlier_ch) if w.outlier_ch is not None else None
    return KvcCache(w.fmt, w.batch, w.hkv, max_tokens or w.max_tokens, page_size=w.page_size,
                    block_table=table, num_pages=w.num_pages, fp16_rows=w.fp16_shadow, kT=w.kT,
                    outlier_ch=oc, outlier_v=w.outlier_v)


def prefill(cache: KvcCache, w):
    """Append every sequence's n_b cached tokens in one call."""
    n_new = dev(w.seq_lens.astype(np.int32))
    cache.append(dev(w.k), dev(w.v), n_new)


def append_step_token(cache: KvcCache, w):
    cache.append(dev(w.k_new), dev(w.v_new))


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = ~(np.abs(gpu - ref) <= atol + rtol * np.abs(ref))
    bad &= ~(np.isneginf(gpu) & np.isneginf(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        worst = np.abs(gpu - ref)[bad].max()
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance "
                             f"(worst abs err {worst:.3g}); first at {idx.tolist()}: "
                             f"gpu {gpu[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
