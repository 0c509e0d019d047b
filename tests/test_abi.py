"""C-ABI library: loads, exports every declared symbol, rejects bad arguments on the host.

CPU only: every call below fails validation before any HIP call, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from decode_attention_sparse_kvc_amd import kvc
from kvc_layout import check_bit_tables

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = kvc.lib()
    names = declared_functions()
    assert {"kvc_quantize_append", "kvc_score_topk", "kvc_attend_decode", "kvc_accum_scores",
            "kvc_topk_mass", "kvc_workspace_bytes", "kvc_status_str", "kvc_abi_version",
            "kvc_build_digest"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert kvc.kvc_abi_version() == kvc.ABI_VERSION


def test_status_strings():
    for s in range(6):
        assert kvc.kvc_status_str(s) and "unknown" not in kvc.kvc_status_str(s)
    assert "unknown" in kvc.kvc_status_str(99)


def test_struct_field_count_matches_header():
    text = open(HEADER).read()
    body = text[text.index("typedef struct kvc_cache {"):text.index("} kvc_cache;")]
    fields = [l for l in body.splitlines()[1:] if ";" in l]
    assert len(fields) == len(kvc.kvc_cache._fields_)
    for line, (name, _) in zip(fields, kvc.kvc_cache._fields_):
        assert re.search(r"\b%s\s*;" % name, line), (line, name)


def _desc(**kw):
    d = kvc.kvc_cache()
    base = dict(abi_version=kvc.ABI_VERSION, format=1, batch=1, num_kv_heads=1, head_dim=128, group_size=64,
                page_size=0, max_tokens=64, max_pages=0, num_pages=0,
                seq_lens=0x1000, k_codes=0x2000, v_codes=0x3000, k_meta=0x4000, v_meta=0x5000,
                k_tail=0x6000, v_tail=0x7000, k_absmax=0x8000)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


BAD = [
    (dict(abi_version=1), 1), (dict(format=7), 3), (dict(head_dim=64), 3), (dict(group_size=32), 3),
    (dict(batch=0), 2), (dict(max_tokens=100), 2), (dict(seq_lens=None), 1),
    (dict(k_codes=None), 1), (dict(k_meta=0x4004), 1), (dict(k_codes=0x2008), 1),
    (dict(page_size=8, max_tokens=64, max_pages=8, num_pages=8, block_table=0x9000), 2),
    (dict(format=2, page_size=16, max_tokens=64, max_pages=4, num_pages=4, block_table=0x9000), 2),
    (dict(page_size=16, max_tokens=64, max_pages=2, num_pages=4, block_table=0x9000), 2),
    (dict(page_size=16, max_tokens=64, max_pages=4, num_pages=4), 1),
    (dict(format=0), 1),   # fp16 cache without k16/v16
    (dict(n_outlier=5, outlier_ch=0xA000, k_outlier=0xB000), 1),
    (dict(n_outlier=-1), 1),
    (dict(n_outlier=2, outlier_ch=0xA000), 1),                        # no outlier store
    (dict(n_outlier=2, outlier_ch=0xA004, k_outlier=0xB000), 1),      # misaligned list
    (dict(n_outlier=2, outlier_ch=0xA000, k_outlier=0xB004), 1),      # misaligned store
    (dict(n_outlier=2, outlier_ch=0xA000, k_outlier=0xB000, v_outlier=0xC002), 1),
    (dict(format=2, n_outlier=1, outlier_ch=0xA000, k_outlier=0xB000), 3),   # INT4 only
]


@pytest.mark.parametrize("kw,status", BAD)
def test_quantize_append_rejects_bad_descriptors(kw, status):
    d = _desc(**kw)
    st = kvc.lib().kvc_quantize_append(ctypes.byref(d), 0x10000, 0x20000, None, 1, None, None)
    assert st == status


def test_quantize_append_argument_checks():
    d = _desc()
    L = kvc.lib()
    assert L.kvc_quantize_append(None, 0x10000, 0x20000, None, 1, None, None) == 1
    assert L.kvc_quantize_append(ctypes.byref(d), None, 0x20000, None, 1, None, None) == 1
    assert L.kvc_quantize_append(ctypes.byref(d), 0x10008, 0x20000, None, 1, None, None) == 1
    assert L.kvc_quantize_append(ctypes.byref(d), 0x10000, 0x20000, None, 65, None, None) == 2
    assert L.kvc_quantize_append(ctypes.byref(d), 0x10000, 0x20000, None, -1, None, None) == 2
    assert L.kvc_quantize_append(ctypes.byref(d), 0x10000, 0x20000, None, 0, None, None) == 0


def test_packing_tables_are_permutations():
    check_bit_tables()


def test_score_topk_and_accum_argument_checks():
    d = _desc(format=0, k16=0x10000, v16=0x20000, k_codes=None, v_codes=None, k_meta=None,
              v_meta=None, k_tail=None, v_tail=None)
    L = kvc.lib()
    ok = dict(q=0x30000, hq=8, mode=1, n_crit=8, ext=None, sink=0, win=0, kps=None, kmax=4,
              idx=0x40000, sc=None, ch=None, ws=0x50000, wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return L.kvc_score_topk(ctypes.byref(d), a["q"], a["hq"], a["mode"], a["n_crit"], a["ext"],
                                a["sink"], a["win"], a["kps"], a["kmax"], a["idx"], a["sc"],
                                a["ch"], a["ws"], a["wsb"], None)
    assert call(hq=0) == 2
    assert call(hq=17) == 3              # more than 16 query heads per KV head
    assert call(mode=5) == 1
    assert call(n_crit=0) == 1 and call(n_crit=129) == 1
    assert call(kmax=-1) == 1 and call(sink=-1) == 1
    assert call(idx=None) == 1
    assert call(wsb=16) == 4 and call(ws=None) == 4
    assert call(mode=2) == 1             # external scores need ext
    assert call(mode=1 | 16, kmax=0) == 0   # block ranking is a flag on a score mode
    assert call(mode=3 | 16) == 1 and call(mode=32) == 1
    assert call(kmax=0) == 0             # nothing to select: no launch
    d.k_absmax = None
    assert call() == 1                   # critical channels need max|K|
    assert L.kvc_accum_scores(ctypes.byref(d), 1, 0x60000, 7, 0x70000, 1, 0x80000, 4, 2, 2, 0x90000, None) == 2
    assert L.kvc_accum_scores(ctypes.byref(d), 1, None, 100, 0x70000, 0, None, 0, 0, 0, 0x90000, None) == 1


def test_workspace_sizes():
    d = _desc(max_tokens=4096)
    L = kvc.lib()
    a1 = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0)
    a2 = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 1, 128, 4, 64)
    t = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, d, 4)
    assert a1 > 0 and a2 > 0 and t >= 4096 * 8
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 7, 0, 0, 0) == 0      # bad mode
    a3 = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 3, 61, 4, 64)          # blocks mode
    assert a3 > 0
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 36, 0, 0, 0, 0) == 0     # G = 36 > 8
    # the planned workgroup count is an explicit argument: 0 is the default plan,
    # more workgroups mean more split partials, out-of-range values are rejected
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0, 0) == a1
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0, 1) < a1
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0, 4096) >= a1
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0, -1) == 0
    assert kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 4, 0, 0, 0, 0, 65537) == 0


def test_topk_mass_argument_checks():
    d = _desc(max_tokens=4096, num_kv_heads=2)
    L = kvc.lib()

    need = kvc.kvc_workspace_bytes(kvc.OP_TOPK_MASS, d, 8)
    assert need > 0 and kvc.kvc_workspace_bytes(kvc.OP_TOPK_MASS, d, 3) == 0

    def call(hq=8, logits=0x10000, stride=4096, lse=0x20000, k=16, out=0x30000, ws=0x40000, nb=None):
        return L.kvc_topk_mass(ctypes.byref(d), hq, logits, stride, lse, k, out, ws,
                               need if nb is None else nb, None)
    assert call(hq=0) == 2 and call(hq=3) == 2
    assert call(logits=None) == 1 and call(lse=None) == 1 and call(out=None) == 1
    assert call(logits=0x10002) == 1
    assert call(k=-1) == 1
    assert call(stride=4095) == 2
    assert call(ws=None) == 4 and call(ws=0x40008) == 4 and call(nb=need - 1) == 4


def test_library_digest_names_its_sources():
    """The loaded library was compiled from the sources beside it (a stale build is refused)."""
    from decode_attention_sparse_kvc_amd.build import source_digest
    assert kvc.kvc_build_digest() == source_digest()
    assert len(source_digest()) == 16


def test_noalloc_rejects_calls_beyond_its_scratch():
    """kvc_attend_decode_noalloc refuses a call whose workspace exceeds the static scratch,
    before any device work (so this runs without a GPU); its other checks are the
    workspace call's."""
    L = kvc.lib()
    # 64 sequences x 64K tokens, keep mode: the row plan alone exceeds 32 MiB
    d = _desc(batch=64, num_kv_heads=8, max_tokens=65536, k16=0x100000, v16=0x200000)
    need = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, d, 32, 2, 20000, 4, 2048)
    assert need > kvc.NOALLOC_SCRATCH_BYTES
    st = L.kvc_attend_decode_noalloc(ctypes.byref(d), 0x30000, 32, 0.088, 2, 0x40000, 20000, 4,
                                     2048, 0x50000, 0x60000, None, 0, None)
    assert st == 6 and "static scratch" in kvc.kvc_status_str(6)
    assert L.kvc_attend_decode_noalloc(None, 0x30000, 32, 0.088, 0, None, 0, 0, 0, 0x50000,
                                       0x60000, None, 0, None) == 1
    assert L.kvc_attend_decode_noalloc(ctypes.byref(d), 0x30000, 32, 0.0, 0, None, 0, 0, 0,
                                       0x50000, 0x60000, None, 0, None) == 1
