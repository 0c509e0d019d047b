"""Host logic of the benchmark (CPU only): the algorithmic bytes a call moves, the
refusal of more than one GPU, and the source-digest gate on counter summaries."""
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _w(fmt="int4", mode="dense", hq=32, hkv=8, batch=1, n_sink=0, n_window=0, top_k=None,
       accumulate=False, prefer_k=0, outlier_ch=None, outlier_v=True):
    return types.SimpleNamespace(fmt=fmt, mode=mode, hq=hq, hkv=hkv, batch=batch, n_sink=n_sink,
                                 n_window=n_window, top_k=top_k, accumulate=accumulate,
                                 prefer_k=prefer_k, outlier_ch=outlier_ch, outlier_v=outlier_v)


QO = 32 * 128 * 2 + 32 * 129 * 4     # q, out and lse of one 32-head sequence


def test_dense_bytes_per_format():
    """Per token per KV head: INT4 144 B, 1-bit 48 B, FP8 256 B, fp16 512 B; the
    incomplete last group of a quantized cache is read as fp16 rows."""
    n = 131072
    assert bench.attend_bytes(_w("int4"), [n], None) == 8 * n * 144 + QO
    assert bench.attend_bytes(_w("int1"), [n], None) == 8 * n * 48 + QO
    assert bench.attend_bytes(_w("fp8"), [n], None) == 8 * n * 256 + QO
    assert bench.attend_bytes(_w("fp16"), [n], None) == 8 * n * 512 + QO
    assert bench.attend_bytes(_w("int4"), [n + 1], None) == 8 * (n * 144 + 512) + QO
    assert bench.attend_bytes(_w("fp8"), [n + 1], None) == 8 * (n + 1) * 256 + QO


def test_outlier_store_bytes():
    ch = np.zeros((8, 3), np.int32)
    n = 4096
    assert bench.attend_bytes(_w(outlier_ch=ch, outlier_v=False), [n], None) == 8 * n * 152 + QO
    assert bench.attend_bytes(_w(outlier_ch=ch), [n], None) == 8 * n * 160 + QO


def test_sparse_bytes():
    """Drop: sinks + selected + window rows; blocks: 64 rows per kept block; keep:
    fp16 keep set + codes for the rest; logits written when accumulating."""
    n, k = 131072, 4096
    top = np.array([k])
    drop = _w("fp16", "drop", top_k=top)
    assert bench.attend_bytes(drop, [n], [k]) == 8 * k * 512 + QO
    drop_acc = _w("fp16", "drop", top_k=top, accumulate=True)
    assert bench.attend_bytes(drop_acc, [n], [k]) == 8 * k * 512 + 32 * k * 4 + QO
    blocks = _w("int4", "blocks", n_sink=4, n_window=100, top_k=np.array([61]))
    assert bench.attend_bytes(blocks, [n], [61]) == 8 * (4 + 64 * 61 + 100) * 144 + QO
    keep = _w("int4", "keep", n_sink=4, n_window=2048, top_k=np.array([n // 5]))
    kept = 4 + n // 5 + 2048
    assert bench.attend_bytes(keep, [n], [n // 5]) == 8 * (kept * 512 + (n - kept) * 144) + QO


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    """A counter summary is used only while its digest names the built sources."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attend_kernel_wl_pmc.txt").write_text(
        "# header\nhbm_bytes_per_launch: 1234\nsrc_digest: abc\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("attend_kernel", "wl", "abc") == 1234.0
    assert bench.read_traffic("attend_kernel", "wl", "abd") is None
    assert bench.read_traffic("attend_kernel", "other", "abc") is None
