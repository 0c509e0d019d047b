"""Device buffers of one layer's compressed KV cache, laid out as include/kvc.h defines.

Plumbing only: allocates (zero-filled) torch tensors of the sizes the C ABI
expects and fills the ``kvc_cache`` descriptor with their addresses.  All
arithmetic on them happens in the library's kernels.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import kvc

_BYTES_PER_SLOT = {"int4": 64, "int1": 16, "fp8": 128}   # code bytes per token per KV head (K or V)


class KvcCache:
    """Buffers + descriptor.  ``fmt`` in {"fp16", "int4", "int1", "fp8"}.

    page_size 0 is a contiguous cache; otherwise ``block_table`` [B, max_pages]
    (int32, physical page ids) and ``num_pages`` describe the page pools.
    ``fp16_rows``: keep k16/v16 (always true for fp16).  ``kT``: channel-major K.
    ``outlier_ch``: int4 only, [Hkv, m] ascending channels (m <= 4) whose K is
    kept at fp16 in ``k_outlier`` beside the codes (and their V in
    ``v_outlier`` when ``outlier_v``).
    """

    def __init__(self, fmt: str, batch: int, num_kv_heads: int, max_tokens: int,
                 page_size: int = 0, block_table: Optional[torch.Tensor] = None,
                 num_pages: int = 0, fp16_rows: bool = False, kT: bool = False,
                 outlier_ch: Optional[torch.Tensor] = None, outlier_v: bool = True,
                 device="cuda"):
        assert fmt in kvc.FMT
        assert max_tokens % kvc.GROUP == 0
        self.fmt, self.batch, self.hkv, self.max_tokens = fmt, batch, num_kv_heads, max_tokens
        self.page_size, self.num_pages = page_size, num_pages
        self.device = torch.device(device)
        D = kvc.HEAD_DIM
        if page_size > 0:
            assert block_table is not None
            self.block_table = block_table.to(device=self.device, dtype=torch.int32).contiguous()
            self.max_pages = int(self.block_table.shape[1])
            slots = num_pages * num_kv_heads * page_size
        else:
            self.block_table = None
            self.max_pages = 0
            slots = batch * num_kv_heads * max_tokens
        self.slots = slots
        z = dict(device=self.device)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, **z)
        self.k_codes = self.v_codes = self.k_meta = self.v_meta = None
        self.k_tail = self.v_tail = self.k16 = self.v16 = self.kT = None
        if fmt == "fp8":   # E4M3 rows only: no groups, metadata or tail
            self.k_codes = torch.zeros(slots * _BYTES_PER_SLOT[fmt], dtype=torch.uint8, **z)
            self.v_codes = torch.zeros_like(self.k_codes)
        elif fmt != "fp16":
            nb = slots * _BYTES_PER_SLOT[fmt]
            self.k_codes = torch.zeros(nb, dtype=torch.uint8, **z)
            self.v_codes = torch.zeros(nb, dtype=torch.uint8, **z)
            self.k_meta = torch.zeros(batch, num_kv_heads, max_tokens // kvc.GROUP, 2, D,
                                      dtype=torch.float16, **z)
            self.v_meta = torch.zeros(slots, 4, dtype=torch.float16, **z)
            self.k_tail = torch.zeros(batch, num_kv_heads, kvc.GROUP, D, dtype=torch.float16, **z)
            self.v_tail = torch.zeros_like(self.k_tail)
        if fmt == "fp16" or fp16_rows:
            self.k16 = torch.zeros(slots, D, dtype=torch.float16, **z)
            self.v16 = torch.zeros(slots, D, dtype=torch.float16, **z)
        if kT:
            self.kT = torch.zeros(batch, num_kv_heads, D, max_tokens, dtype=torch.float16, **z)
        self.k_absmax = torch.zeros(batch, num_kv_heads, D, dtype=torch.float32, **z)
        self.n_outlier, self.outlier_ch, self.k_outlier, self.v_outlier = 0, None, None, None
        if outlier_ch is not None and outlier_ch.shape[-1] > 0:
            assert fmt == "int4" and outlier_ch.shape[0] == num_kv_heads
            m = int(outlier_ch.shape[-1])
            assert m <= kvc.MAX_OUTLIERS
            ch = torch.zeros(num_kv_heads, kvc.MAX_OUTLIERS, dtype=torch.int32)
            ch[:, :m] = torch.as_tensor(outlier_ch, dtype=torch.int32).cpu()
            self.n_outlier = m
            self.outlier_ch = ch.to(self.device)
            self.k_outlier = torch.zeros(slots, kvc.MAX_OUTLIERS, dtype=torch.float16, **z)
            if outlier_v:
                self.v_outlier = torch.zeros_like(self.k_outlier)
        self._refresh()

    def _refresh(self):
        p = kvc._ptr
        self.desc = kvc.kvc_cache(
            kvc.ABI_VERSION, kvc.FMT[self.fmt], self.batch, self.hkv, kvc.HEAD_DIM, kvc.GROUP,
            self.page_size, self.max_tokens, self.max_pages, self.num_pages,
            p(self.block_table), p(self.seq_lens), p(self.k_codes), p(self.v_codes),
            p(self.k_meta), p(self.v_meta), p(self.k_tail), p(self.v_tail),
            p(self.k16), p(self.v16), p(self.kT), p(self.k_absmax),
            self.n_outlier, p(self.outlier_ch), p(self.k_outlier), p(self.v_outlier))

    def tensors(self):
        names = ["block_table", "seq_lens", "k_codes", "v_codes", "k_meta", "v_meta", "k_tail",
                 "v_tail", "k16", "v16", "kT", "k_absmax", "outlier_ch", "k_outlier", "v_outlier"]
        return {n: getattr(self, n) for n in names if getattr(self, n) is not None}

    def clone(self) -> "KvcCache":
        """An independent copy of every buffer (same descriptor shape)."""
        other = object.__new__(KvcCache)
        other.__dict__.update(self.__dict__)
        for n, t in self.tensors().items():
            setattr(other, n, t.clone())
        other._refresh()
        return other

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors().values())

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, n_new: Optional[torch.Tensor] = None,
               overflow: Optional[torch.Tensor] = None, stream=None):
        """kvc_quantize_append of k_new/v_new [B, n, Hkv, 128] fp16 (contiguous)."""
        assert k_new.dtype == torch.float16 and k_new.is_contiguous() and v_new.is_contiguous()
        assert k_new.shape[0] == self.batch and k_new.shape[2] == self.hkv
        kvc.kvc_quantize_append(self.desc, k_new, v_new, n_new, int(k_new.shape[1]), overflow, stream)


def pages_needed(lengths, page_size: int) -> int:
    return sum(math.ceil(int(n) / page_size) for n in lengths)
