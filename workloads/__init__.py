"""Seeded synthetic inputs for one decode step of attention over a compressed KV cache.

This module is shared by the CPU oracle, the GPU tests and the benchmark.  It
holds random draws, casts to fp16 and index bookkeeping only: no quantization,
scoring, selection, softmax or accumulation arithmetic lives here, so neither
side of a parity check can borrow the other's maths through it.

Every workload is Llama-3.1-8B shaped per layer (32 query heads, 8 KV heads,
head_dim 128) except the single-head correctness case.  The shapes, value laws
and selection parameters follow the problem statement of the TailorKV article
(sections 2.2, 2.3 and 5.1: 64-token quantization groups, 8 critical channels,
a 3% keep ratio), the StreamingLLM/H2O survey (section 3: 4 sink tokens, a
2048-token window, cumulative attention scores) and PagedAttention's 16-token
blocks (same survey, section 1).  The draw order of each workload is part of
its definition and is listed in its docstring.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

HEAD_DIM = 128
GROUP = 64
_BLOCK = 1 << 22          # elements per independently seeded block of a bulk draw


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.

    Arrays are numpy, fp16 data as ``np.float16``:
      k, v      [B, n_max, Hkv, D]  keys/values of the cached context (rows >= n_b unused)
      q         [B, Hq, D]          this step's query
      k_new, v_new [B, 1, Hkv, D]   the token this step appends
      seq_lens  [B] int32           cached context length n_b before the step
      acc       [B, Hkv, n_max] float32 or None   cumulative (H2O) scores
      block_table [B, max_pages] int32 or None    logical->physical 16-token pages
    """
    name: str
    seed: int
    fmt: str                 # "int4" | "int1" | "fp16" | "fp8"
    batch: int
    hq: int
    hkv: int
    k: np.ndarray
    v: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    seq_lens: np.ndarray
    mode: str = "dense"      # attend mode: "dense" | "drop" | "keep" | "blocks"
    score: Optional[str] = None  # "exact" | "critical" | "external" | None
    granule: str = "token"   # what Top-K ranks: "token" or "block" (64-token blocks)
    n_sink: int = 0
    n_window: int = 0
    top_k: Optional[np.ndarray] = None   # [B] int32 tokens to select per sequence
    n_crit: int = 8
    accumulate: bool = False             # H2O update after attending
    acc: Optional[np.ndarray] = None
    page_size: int = 0
    block_table: Optional[np.ndarray] = None
    num_pages: int = 0
    max_tokens: int = 0                  # per-sequence capacity (multiple of 64)
    kT: bool = False                     # keep a channel-major K copy (fp16 caches)
    fp16_shadow: bool = False            # keep full fp16 rows beside quantized codes
    prefer_k: int = 0                    # > 0: also the top-k probability mass of each row
    outlier_ch: Optional[np.ndarray] = None   # [Hkv, m] int4: channels kept at fp16
    outlier_v: bool = True                    # isolate those channels of V too
    planted: Optional[np.ndarray] = None      # [Hkv, m] the K channels the generator scaled

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def n_max(self) -> int:
        return int(self.k.shape[1])

    @property
    def sm_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(HEAD_DIM)))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _bulk_normal(ss: np.random.SeedSequence, shape) -> np.ndarray:
    """float32 N(0,1) array filled in blocks of 2^22 elements (row-major order),
    block i drawn from ``default_rng(ss.spawn(nblocks)[i])``.  The result does
    not depend on how many threads fill it."""
    out = np.empty(shape, np.float32)
    flat = out.reshape(-1)
    nblk = (flat.size + _BLOCK - 1) // _BLOCK
    kids = ss.spawn(nblk)

    def fill(i):
        np.random.default_rng(kids[i]).standard_normal(
            dtype=np.float32, out=flat[i * _BLOCK:(i + 1) * _BLOCK])

    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def _f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even (blockwise, threaded)."""
    out = np.empty(x.shape, np.float16)
    fo, fi = out.reshape(-1), x.reshape(-1)

    def cast(i):
        fo[i * _BLOCK:(i + 1) * _BLOCK] = fi[i * _BLOCK:(i + 1) * _BLOCK]

    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(cast, range((fi.size + _BLOCK - 1) // _BLOCK)))
    return out


def _streams(seed: int):
    """Independent streams of a workload's seed: K bulk, V bulk, everything else."""
    s_k, s_v, s_rest = np.random.SeedSequence(seed).spawn(3)
    return s_k, s_v, np.random.default_rng(s_rest)


def _capacity(n: int, extra: int) -> int:
    need = n + extra
    return ((need + GROUP - 1) // GROUP) * GROUP


def _new_token(rng, batch, hkv):
    k_new = _normal(rng, (batch, 1, hkv, HEAD_DIM)).astype(np.float16)
    v_new = _normal(rng, (batch, 1, hkv, HEAD_DIM)).astype(np.float16)
    return k_new, v_new


def single_head_4k(n_ctx: int = 4096, seed: int = 0) -> Workload:
    """Single head, batch 1, INT4 cache, exact-score Top-128 + 4 sinks + 64-token window.

    Draws: K [1,N,1,D] and V ~ N(0,1) from the seed's K and V bulk streams;
    from the third stream, in order: 4 outlier K channels (choice without
    replacement) scaled by 8, q [1,1,D] ~ N(0,1), the appended token's k, v.
    All cast to fp16 (round to nearest even).
    """
    s_k, s_v, rng = _streams(seed)
    k = _bulk_normal(s_k, (1, n_ctx, 1, HEAD_DIM))
    v = _bulk_normal(s_v, (1, n_ctx, 1, HEAD_DIM))
    out = rng.choice(HEAD_DIM, 4, replace=False)
    k[..., out] *= np.float32(8.0)
    q = _normal(rng, (1, 1, HEAD_DIM))
    k_new, v_new = _new_token(rng, 1, 1)
    return Workload(
        name="single_head_int4_exact_top128", seed=seed, fmt="int4", batch=1, hq=1, hkv=1,
        k=_f16(k), v=_f16(v), q=q.astype(np.float16),
        k_new=k_new, v_new=v_new, seq_lens=np.array([n_ctx], np.int32),
        mode="drop", score="exact", n_sink=4, n_window=64,
        top_k=np.array([128], np.int32), max_tokens=_capacity(n_ctx, 64))


def _llama_dense(name: str, fmt: str, n_ctx: int, seed: int, outliers: bool) -> Workload:
    """32 q heads / 8 KV heads, batch 1, dense decode over every cached token.

    Draws: K [1,N,8,D] and V ~ N(0,1) from the bulk streams; from the third
    stream, in order: if outliers, for each KV head, 3 channels (2% of 128,
    rounded up; choice without replacement) of K scaled by 8; q [1,32,D];
    the appended k, v.
    """
    s_k, s_v, rng = _streams(seed)
    hq, hkv = 32, 8
    k = _bulk_normal(s_k, (1, n_ctx, hkv, HEAD_DIM))
    v = _bulk_normal(s_v, (1, n_ctx, hkv, HEAD_DIM))
    planted = None
    if outliers:
        planted = np.zeros((hkv, 3), np.int32)
        for g in range(hkv):
            out = rng.choice(HEAD_DIM, 3, replace=False)
            k[:, :, g, out] *= np.float32(8.0)
            planted[g] = np.sort(out)
    q = _normal(rng, (1, hq, HEAD_DIM))
    k_new, v_new = _new_token(rng, 1, hkv)
    return Workload(
        name=name, seed=seed, fmt=fmt, batch=1, hq=hq, hkv=hkv,
        k=_f16(k), v=_f16(v), q=q.astype(np.float16),
        k_new=k_new, v_new=v_new, seq_lens=np.array([n_ctx], np.int32),
        mode="dense", max_tokens=_capacity(n_ctx, 64), planted=planted)


def int4_dense(n_ctx: int = 32768, seed: int = 1) -> Workload:
    """INT4 K per-channel / V group-64, dense; 2% outlier K channels x8 (seed 1)."""
    tag = "32k" if n_ctx == 32768 else ("128k" if n_ctx == 131072 else str(n_ctx))
    return _llama_dense(f"llama8b_layer_int4_dense_{tag}", "int4", n_ctx, seed, True)


def int4_outlier_dense(n_ctx: int = 131072, seed: int = 1) -> Workload:
    """The INT4 layer (seed 1) with its outlier K channels kept at fp16 beside the
    codes.  The channel list stands in for the offline variance analysis: it is
    the generator's planted channels (x8, so 64x the variance of the others)."""
    w = int4_dense(n_ctx, seed)
    tag = "32k" if n_ctx == 32768 else ("128k" if n_ctx == 131072 else str(n_ctx))
    w.name = f"llama8b_layer_int4_outlier3_dense_{tag}"
    w.outlier_ch = w.planted.copy()
    return w


def fp8_dense(n_ctx: int = 131072, seed: int = 1) -> Workload:
    """FP8 (E4M3) warm tier: the INT4 layer's draws (seed 1, same outliers) stored
    as E4M3 codes, dense decode."""
    tag = "32k" if n_ctx == 32768 else ("128k" if n_ctx == 131072 else str(n_ctx))
    return _llama_dense(f"llama8b_layer_fp8_dense_{tag}", "fp8", n_ctx, seed, True)


def int1_dense(n_ctx: int = 131072, seed: int = 2) -> Workload:
    """TailorKV quantization-friendly layer: 1-bit K and V, dense decode (seed 2)."""
    tag = "128k" if n_ctx == 131072 else str(n_ctx)
    return _llama_dense(f"llama8b_layer_int1_dense_{tag}", "int1", n_ctx, seed, False)


def sparse_crit8(n_ctx: int = 131072, seed: int = 3, n_planted: int = 512,
                 top_k: int = 4096) -> Workload:
    """Sparsity-friendly fp16 layer with planted key tokens, 8-channel Top-K retrieval.

    Draws: K [1,N,8,D] and V ~ N(0,1) from the bulk streams; from the third
    stream, in order: q [1,32,D]; per KV head g, ``n_planted`` token ids
    (choice without replacement), the j-th assigned to query head 4g + j%4;
    the appended k, v.
    A planted key keeps its norm and is turned to cosine 0.6 with its query:
    k := |k| (0.6 q/|q| + 0.8 u), u the unit part of k orthogonal to q
    (fp64, then fp16).
    """
    s_k, s_v, rng = _streams(seed)
    hq, hkv = 32, 8
    k = _bulk_normal(s_k, (1, n_ctx, hkv, HEAD_DIM))
    v = _bulk_normal(s_v, (1, n_ctx, hkv, HEAD_DIM))
    q = _normal(rng, (1, hq, HEAD_DIM)).astype(np.float16)
    qf = q.astype(np.float64)
    for g in range(hkv):
        ids = rng.choice(n_ctx, n_planted, replace=False)
        for j, t in enumerate(ids):
            h = 4 * g + (j % 4)
            qh = qf[0, h] / np.linalg.norm(qf[0, h])
            kt = k[0, t, g].astype(np.float64)
            perp = kt - np.dot(kt, qh) * qh
            perp /= np.linalg.norm(perp)
            k[0, t, g] = (np.linalg.norm(kt) * (0.6 * qh + 0.8 * perp)).astype(np.float32)
    k_new, v_new = _new_token(rng, 1, hkv)
    tag = "128k" if n_ctx == 131072 else str(n_ctx)
    return Workload(
        name=f"llama8b_layer_fp16_crit8_top{top_k}_{tag}", seed=seed, fmt="fp16",
        batch=1, hq=hq, hkv=hkv,
        k=_f16(k), v=_f16(v), q=q,
        k_new=k_new, v_new=v_new, seq_lens=np.array([n_ctx], np.int32),
        mode="drop", score="critical", n_sink=0, n_window=0,
        top_k=np.array([top_k], np.int32), n_crit=8, accumulate=True,
        acc=np.zeros((1, hkv, _capacity(n_ctx, 64)), np.float32),
        max_tokens=_capacity(n_ctx, 64), kT=True)


def sparse_blocks(n_ctx: int = 131072, fmt: str = "fp16", top_blocks: int = 61,
                  seed: int = 3) -> Workload:
    """Block-granular selection on the sparsity-friendly layer: the draws of
    ``sparse_crit8`` (same seed, same order), scored on 8 critical channels,
    ranked by the mean score of each 64-token block, the top ``top_blocks``
    blocks kept (61 = 3% of the 2048 blocks at 128K), then attended (with the
    H2O update).  fmt "int4" stores the same keys and values as INT4 codes."""
    w = sparse_crit8(n_ctx, seed=seed, n_planted=min(512, n_ctx))
    tag = "128k" if n_ctx == 131072 else str(n_ctx)
    w.name = f"llama8b_layer_{fmt}_crit8_block{top_blocks}_{tag}"
    w.fmt = fmt
    w.mode = "blocks"
    w.granule = "block"
    w.top_k = np.array([top_blocks], np.int32)
    w.kT = fmt == "fp16"
    return w


def batched_joint(batch: int = 16, lo: int = 8192, hi: int = 32768, seed: int = 4,
                  page: int = 16, n_sink: int = 4, n_window: int = 2048) -> Workload:
    """Batched joint compression over a paged INT4 cache with an fp16 keep set.

    Draws: from the third stream, n_b for each sequence ~ uniform integers in
    [lo, hi]; K and V [B, max n_b, 8, D] ~ N(0,1) from the bulk streams; then
    from the third stream, in order: q [B,32,D] ~ N(0,1); cumulative scores
    acc [B, 8, capacity] ~ lognormal(0, 1.5) (zeroed at and beyond n_b); a
    permutation of all physical pages, handed out to sequences in order, one
    page per 16 tokens of capacity n_b + 1; the appended k, v.
    The keep set per (sequence, KV head) is 4 sinks, the last 2048 tokens and
    the top floor(n_b / 5) of the tokens in between by cumulative score.
    """
    s_k, s_v, rng = _streams(seed)
    hq, hkv = 32, 8
    n = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    n_max = int(n.max())
    k = _bulk_normal(s_k, (batch, n_max, hkv, HEAD_DIM))
    v = _bulk_normal(s_v, (batch, n_max, hkv, HEAD_DIM))
    q = _normal(rng, (batch, hq, HEAD_DIM))
    cap = _capacity(n_max, 64)
    acc = rng.lognormal(0.0, 1.5, size=(batch, hkv, cap)).astype(np.float32)
    for b in range(batch):
        acc[b, :, n[b]:] = 0.0
    pages_per = [(int(nb) + 1 + page - 1) // page for nb in n]
    total = int(sum(pages_per))
    perm = rng.permutation(total).astype(np.int32)
    max_pages = cap // page
    table = np.full((batch, max_pages), -1, np.int32)
    pos = 0
    for b in range(batch):
        table[b, :pages_per[b]] = perm[pos:pos + pages_per[b]]
        pos += pages_per[b]
    k_new, v_new = _new_token(rng, batch, hkv)
    return Workload(
        name=f"batch{batch}_ragged_paged_int4_keep_fp16", seed=seed, fmt="int4",
        batch=batch, hq=hq, hkv=hkv,
        k=_f16(k), v=_f16(v), q=q.astype(np.float16),
        k_new=k_new, v_new=v_new, seq_lens=n,
        mode="keep", score="external", n_sink=n_sink, n_window=n_window,
        top_k=(n // 5).astype(np.int32), accumulate=True, acc=acc,
        page_size=page, block_table=table, num_pages=total, max_tokens=cap,
        fp16_shadow=True)


# Full-size workloads by name (the benchmark and the full-size parity tests).
def _with_prefer(w: Workload, k: int) -> Workload:
    """The same layer with the dense preference score's top-k mass per row
    (TailorKV article, section 2.1) computed from the step's attention."""
    w.prefer_k = k
    w.name += f"_topmass{k}"
    return w


FULL = {
    "single_head_int4_exact_top128": lambda: single_head_4k(),
    "llama8b_layer_int4_dense_32k": lambda: int4_dense(32768),
    "llama8b_layer_int4_dense_128k": lambda: int4_dense(131072),
    "llama8b_layer_int1_dense_128k": lambda: int1_dense(131072),
    "llama8b_layer_fp16_crit8_top4096_128k": lambda: sparse_crit8(131072),
    "batch16_ragged_paged_int4_keep_fp16": lambda: batched_joint(),
    "llama8b_layer_fp16_crit8_block61_128k": lambda: sparse_blocks(131072, "fp16"),
    "llama8b_layer_int4_crit8_block61_128k": lambda: sparse_blocks(131072, "int4"),
    "llama8b_layer_fp8_dense_128k": lambda: fp8_dense(131072),
    "llama8b_layer_int4_outlier3_dense_128k": lambda: int4_outlier_dense(131072),
    "llama8b_layer_int1_dense_128k_topmass3pct": lambda: _with_prefer(int1_dense(131072), 3932),
}
