"""MI355X-native decode attention over a jointly sparsified + quantized KV cache.

The work is done by ``libkvc.so`` (HIP kernels for gfx950, C ABI in
``include/kvc.h``); this package holds its Python binding (``kvc``) and the
allocation of cache buffers in the ABI's layout (``cache``).
"""
from . import kvc
from .cache import KvcCache
from .kvc import (KvcError, kvc_accum_scores, kvc_attend_decode, kvc_quantize_append,
                  kvc_score_topk, kvc_status_str, kvc_workspace_bytes)

__all__ = ["kvc", "KvcCache", "KvcError", "kvc_quantize_append", "kvc_score_topk",
           "kvc_attend_decode", "kvc_accum_scores", "kvc_workspace_bytes", "kvc_status_str"]
