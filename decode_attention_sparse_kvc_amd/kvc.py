"""Thin Python binding of the kvc C ABI (include/kvc.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libkvc.so.  Functions carry the C names and take torch tensors (or
None for NULL); fp16 data is passed as the tensors' raw bits.  A non-zero
status raises ``KvcError``.  If the library is missing it is built in-tree; a
library whose embedded source digest differs from the sources beside it is
refused (rebuild it with ``build.build()``); if it cannot be loaded, the first
call fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvc.so")

ABI_VERSION = 4
HEAD_DIM = 128
GROUP = 64
MAX_OUTLIERS = 4
FMT = {"fp16": 0, "int4": 1, "int1": 2, "fp8": 3}
SCORE = {"exact": 0, "critical": 1, "external": 2}
SCORE_BLOCKS = 16   # OR'ed into a score mode: rank 64-token blocks
MODE = {"dense": 0, "drop": 1, "keep": 2, "blocks": 3}
OP_SCORE_TOPK, OP_ATTEND, OP_TOPK_MASS = 1, 2, 3
NOALLOC_SCRATCH_BYTES = 32 << 20   # KVC_NOALLOC_SCRATCH_BYTES


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({kvc_status_str(status)})")
        self.status = status


class kvc_cache(ctypes.Structure):
    """Mirror of ``struct kvc_cache`` (include/kvc.h)."""
    _fields_ = [
        ("abi_version", c_int32), ("format", c_int32), ("batch", c_int32),
        ("num_kv_heads", c_int32), ("head_dim", c_int32), ("group_size", c_int32),
        ("page_size", c_int32), ("max_tokens", c_int32), ("max_pages", c_int32),
        ("num_pages", c_int32),
        ("block_table", c_void_p), ("seq_lens", c_void_p),
        ("k_codes", c_void_p), ("v_codes", c_void_p),
        ("k_meta", c_void_p), ("v_meta", c_void_p),
        ("k_tail", c_void_p), ("v_tail", c_void_p),
        ("k16", c_void_p), ("v16", c_void_p), ("kT", c_void_p),
        ("k_absmax", c_void_p),
        ("n_outlier", c_int32), ("outlier_ch", c_void_p), ("k_outlier", c_void_p),
        ("v_outlier", c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from .build import build
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER(kvc_cache)
    lib.kvc_build_digest.restype = ctypes.c_char_p
    from .build import source_digest
    built, here = lib.kvc_build_digest().decode(), source_digest()
    if built != here:
        raise ImportError(f"{LIB_PATH} was built from other sources (digest {built}, sources {here}); "
                          "rebuild it: python -m decode_attention_sparse_kvc_amd.build")
    lib.kvc_abi_version.restype = c_int32
    lib.kvc_status_str.restype = ctypes.c_char_p
    lib.kvc_status_str.argtypes = [c_int32]
    lib.kvc_quantize_append.restype = c_int32
    lib.kvc_quantize_append.argtypes = [P, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
    lib.kvc_score_topk.restype = c_int32
    lib.kvc_score_topk.argtypes = [P, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                   c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]
    lib.kvc_attend_decode.restype = c_int32
    lib.kvc_attend_decode.argtypes = [P, c_void_p, c_int32, c_float, c_int32, c_void_p, c_int32,
                                      c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int64,
                                      c_int32, c_void_p, c_size_t, c_void_p]
    lib.kvc_attend_decode_noalloc.restype = c_int32
    lib.kvc_attend_decode_noalloc.argtypes = [P, c_void_p, c_int32, c_float, c_int32, c_void_p,
                                              c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                              c_void_p, c_int64, c_void_p]
    lib.kvc_accum_scores.restype = c_int32
    lib.kvc_accum_scores.argtypes = [P, c_int32, c_void_p, c_int64, c_void_p, c_int32, c_void_p,
                                     c_int32, c_int32, c_int32, c_void_p, c_void_p]
    lib.kvc_topk_mass.restype = c_int32
    lib.kvc_topk_mass.argtypes = [P, c_int32, c_void_p, c_int64, c_void_p, c_int32, c_void_p,
                                  c_void_p, c_size_t, c_void_p]
    lib.kvc_stream_read.restype = c_int32
    lib.kvc_stream_read.argtypes = [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]
    lib.kvc_workspace_bytes.restype = c_size_t
    lib.kvc_workspace_bytes.argtypes = [c_int32, P, c_int32, c_int32, c_int32, c_int32, c_int32,
                                        c_int32]
    if lib.kvc_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {lib.kvc_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def lib():
    return _load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise KvcError(fn, status)


def kvc_abi_version() -> int:
    return lib().kvc_abi_version()


def kvc_build_digest() -> str:
    return lib().kvc_build_digest().decode()


def kvc_status_str(status: int) -> str:
    return lib().kvc_status_str(status).decode()


def kvc_quantize_append(cache, k_new, v_new, n_new, n_new_max: int, overflow=None, stream=None):
    _check("kvc_quantize_append", lib().kvc_quantize_append(
        ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(n_new), n_new_max, _ptr(overflow),
        _stream(stream)))


def kvc_score_topk(cache, q, num_q_heads: int, score_mode: int, n_crit: int, ext,
                   n_sink: int, n_window: int, k_per_seq, k_max: int, out_idx,
                   out_scores=None, out_channels=None, workspace=None, workspace_bytes: int = 0,
                   stream=None):
    _check("kvc_score_topk", lib().kvc_score_topk(
        ctypes.byref(cache), _ptr(q), num_q_heads, score_mode, n_crit, _ptr(ext), n_sink, n_window,
        _ptr(k_per_seq), k_max, _ptr(out_idx), _ptr(out_scores), _ptr(out_channels),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def kvc_attend_decode(cache, q, num_q_heads: int, sm_scale: float, mode: int, sel, k_max: int,
                      n_sink: int, n_window: int, out, lse, logits=None, logits_stride: int = 0,
                      workspace=None, workspace_bytes: int = 0, stream=None, *,
                      workgroups: int = 0):
    _check("kvc_attend_decode", lib().kvc_attend_decode(
        ctypes.byref(cache), _ptr(q), num_q_heads, sm_scale, mode, _ptr(sel), k_max, n_sink,
        n_window, _ptr(out), _ptr(lse), _ptr(logits), logits_stride, workgroups, _ptr(workspace),
        workspace_bytes, _stream(stream)))


def kvc_attend_decode_noalloc(cache, q, num_q_heads: int, sm_scale: float, mode: int, sel,
                              k_max: int, n_sink: int, n_window: int, out, lse, logits=None,
                              logits_stride: int = 0, stream=None):
    _check("kvc_attend_decode_noalloc", lib().kvc_attend_decode_noalloc(
        ctypes.byref(cache), _ptr(q), num_q_heads, sm_scale, mode, _ptr(sel), k_max, n_sink,
        n_window, _ptr(out), _ptr(lse), _ptr(logits), logits_stride, _stream(stream)))


def kvc_accum_scores(cache, num_q_heads: int, logits, logits_stride: int, lse, mode: int, sel,
                     k_max: int, n_sink: int, n_window: int, acc, stream=None):
    _check("kvc_accum_scores", lib().kvc_accum_scores(
        ctypes.byref(cache), num_q_heads, _ptr(logits), logits_stride, _ptr(lse), mode, _ptr(sel),
        k_max, n_sink, n_window, _ptr(acc), _stream(stream)))


def kvc_topk_mass(cache, num_q_heads: int, logits, logits_stride: int, lse, k: int, out,
                  workspace=None, workspace_bytes: int = 0, stream=None):
    _check("kvc_topk_mass", lib().kvc_topk_mass(
        ctypes.byref(cache), num_q_heads, _ptr(logits), logits_stride, _ptr(lse), k, _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def kvc_stream_read(src, nbytes: int, sink, workgroups: int, stream=None):
    _check("kvc_stream_read", lib().kvc_stream_read(_ptr(src), nbytes, _ptr(sink), workgroups,
                                                    _stream(stream)))


def kvc_workspace_bytes(op: int, cache, num_q_heads: int, mode: int = 0, k_max: int = 0,
                        n_sink: int = 0, n_window: int = 0, workgroups: int = 0) -> int:
    return int(lib().kvc_workspace_bytes(op, ctypes.byref(cache), num_q_heads, mode, k_max,
                                         n_sink, n_window, workgroups))
