#!/usr/bin/env python3
"""Decode attention over a compressed KV cache on one MI355X: throughput + roofline.

One step is the decode hot path of the chosen workload on one synthetic batch,
with the cache already resident in HBM:
  * dense layers (INT4 / 1-bit):  kvc_quantize_append(1 token) + kvc_attend_decode;
  * sparse / joint layers:        + kvc_score_topk before and kvc_accum_scores
                                   after attending.
``value`` is context tokens attended per second for the whole layer (all KV
heads, all sequences).  Cache replicas are rotated so that the working set
exceeds the 256 MB Infinity Cache and bytes come from HBM.

The default run (the INT4 layer at 128K) also times, in the same process,
the second gated call -- the 1-bit 128K layer's kvc_attend_decode -- under
``roofline.gates``, a plain streaming read of the replica buffer
(kvc_stream_read) under ``roofline.ceiling``, and the CPU oracle's attention
leg on the host's cores under ``cpu_baseline``.

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: the benchmark runs on
one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "llama8b_layer_int4_dense_128k"
CODE_BYTES = {"int4": 144, "int1": 48, "fp8": 256}   # per token per KV head, incl. amortized K meta
GRAPH_CALLS = 8                             # at least this many steps (or calls) per replayed graph


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--replica-bytes", type=float, default=1.5 * 2**30,
                    help="total bytes of rotated cache replicas (defeats the Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gates", action="store_true",
                    help="default workload: skip the second gated call (1-bit 128K attend)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="workgroups the attend call is planned for (0: the library default)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every call from Python instead of replaying HIP graphs")
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def src_digest() -> str:
    """Digest of the sources the attend call is built from (its kernels, their
    shared header and the ABI header): counter summaries taken with other
    sources stay valid for it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_sparse_kvc_amd", "csrc")
    for path in (os.path.join(csrc, "attend.hip"), os.path.join(csrc, "internal.h"),
                 os.path.join(ROOT, "include", "kvc.h")):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + f.read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain 1 GiB device-to-device copy, 20 times (for FETCH_SIZE / WRITE_SIZE scaling)."""
    import torch
    n = 2**30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(20):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 20}))


def attend_bytes(w, lens, k_sel) -> int:
    """Algorithmic bytes of one kvc_attend_decode: every byte of the attended
    K/V (codes + metadata, or fp16 rows), q, out, lse and logits written."""
    fmt, hkv, hq, B = w.fmt, w.hkv, w.hq, w.batch
    total = 0
    # quantized tokens of a cache with outlier channels also read their
    # 8-byte outlier-store entries (K, and V when isolated)
    extra = 0 if w.outlier_ch is None else (16 if w.outlier_v else 8)
    code = dict(CODE_BYTES, int4=CODE_BYTES["int4"] + extra)
    for b, n in enumerate(lens):
        n = int(n)
        nq = (n // 64) * 64 if fmt != "fp8" else n     # fp8 has no fp16 tail
        if w.mode == "dense":
            per_head = nq * code[fmt] + (n - nq) * 512 if fmt != "fp16" else n * 512
        elif w.mode == "drop":
            w0 = max(n - w.n_window, min(w.n_sink, n))
            attended = min(w.n_sink, n) + int(k_sel[b]) + (n - w0)
            per_head = attended * (512 if fmt == "fp16" else code[fmt])
        elif w.mode == "blocks":   # k_sel blocks of 64 tokens (every candidate range holds them)
            w0 = max(n - w.n_window, min(w.n_sink, n))
            attended = min(w.n_sink, n) + 64 * int(k_sel[b]) + (n - w0)
            per_head = attended * (512 if fmt == "fp16" else code[fmt])
        else:   # keep: fp16 keep set, codes for the rest (tail rows fp16)
            w0 = max(n - w.n_window, min(w.n_sink, n))
            keep = min(w.n_sink, n) + int(k_sel[b]) + (n - w0)
            rest = n - keep
            per_head = keep * 512 + rest * code[fmt]
        total += hkv * per_head
        if w.accumulate or w.prefer_k:            # logits written
            if w.mode == "drop":
                pos = w.n_sink + int(w.top_k.max()) + w.n_window
            elif w.mode == "blocks":
                pos = w.n_sink + 64 * int(w.top_k.max()) + w.n_window
            else:
                pos = n
            total += hq * pos * 4
    total += B * hq * 128 * 2           # q
    total += B * hq * (128 + 1) * 4     # out + lse
    return total


def read_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if current."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("src_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seconds: float, runs: int = 3):
    """The oracle's attention leg on host cores: for each (sequence, KV head)
    pair, dequantize its cached tokens (oracle.step.token_rows) and attend its
    query group over them (oracle.attend.attend_group) -- the work one
    kvc_attend_decode call does.  The pair caches are built before timing (the
    GPU step does not re-quantize the context either).  Timed on one thread
    over a bounded subset of pairs, and on every core of the affinity mask
    (one pair per thread, BLAS single-threaded) over all pairs; median of
    `runs` runs each, scaled to context tokens per second of the layer."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    from oracle import attend as A
    from oracle import select as S
    from oracle import step as ST
    cores = len(os.sched_getaffinity(0))
    pairs = [(b, g) for b in range(w.batch) for g in range(w.hkv)]
    G = w.group
    if w.mode not in ("dense",):
        raise ValueError("cpu_baseline times dense layers")
    ctx = sum(int(w.seq_lens[b]) for b in range(w.batch))

    def build(p):
        b, g = p
        n = int(w.seq_lens[b])
        oc = None if getattr(w, "outlier_ch", None) is None else w.outlier_ch[g]
        return ST.build_head_cache(w.k[b, :n, g], w.v[b, :n, g], w.fmt, oc,
                                   getattr(w, "outlier_v", True))

    def leg(i):
        b, g = pairs[i]
        keys, vals = ST.token_rows(hcs[i])
        toks = S.attended_tokens("dense", hcs[i].n, 0, 0, None)
        A.attend_group(w.q[b, g * G:(g + 1) * G], keys[toks], vals[toks], w.sm_scale)

    with threadpool_limits(limits=1):
        workers = max(1, min(cores, len(pairs)))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            hcs = list(ex.map(build, pairs))
        # one thread: as many pairs as fit about `seconds` / runs (at least one)
        t0 = time.perf_counter()
        leg(0)
        one = time.perf_counter() - t0
        m = max(1, min(len(pairs), int(seconds / max(runs, 1) / max(one, 1e-3))))
        single = []
        for _ in range(runs):
            t0 = time.perf_counter()
            for i in range(m):
                leg(i)
            single.append(time.perf_counter() - t0)
        # every core: all pairs, one per thread
        multi = []
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            for _ in range(runs):
                t0 = time.perf_counter()
                list(ex.map(leg, range(len(pairs))))
                multi.append(time.perf_counter() - t0)
    t1 = sorted(single)[len(single) // 2]
    tm = sorted(multi)[len(multi) // 2]
    v1 = ctx * (m / len(pairs)) / t1
    vm = ctx / tm
    return {
        "value": vm,
        "unit": "context-tokens/s",
        "cores": workers,
        "kind": "oracle",
        "value_1thread": v1,
        "cores_available": cores,
        "sample": f"attention leg of kvc_attend_decode (dequantize the cached codes, fp64 softmax "
                  f"attention of the query group) per (sequence, KV head) pair, caches prebuilt; "
                  f"all {len(pairs)} pairs on {workers} threads (one pair a thread, "
                  f"{cores} cores in the affinity mask) and {m} pair(s) on 1 thread scaled by "
                  f"{m}/{len(pairs)}; median of {runs} runs ({tm:.2f} s and {t1:.2f} s)",
    }


def make_caches(w, args, extra: int):
    """The workload's cache, prefilled on the GPU, and copies of it: enough
    replicas that rotating over them exceeds args.replica_bytes (defeats the
    256 MB Infinity Cache).  Capacity leaves room for `extra` appended tokens."""
    import numpy as np
    import torch
    from decode_attention_sparse_kvc_amd import KvcCache
    dev = torch.device("cuda")
    cap = ((int(w.seq_lens.max()) + extra + 63) // 64) * 64
    table, num_pages = None, 0
    if w.page_size:   # shuffled pages covering the grown capacity of every sequence
        per = cap // w.page_size
        num_pages = w.batch * per
        perm = np.random.default_rng(w.seed).permutation(num_pages).astype(np.int32)
        table = torch.from_numpy(perm.reshape(w.batch, per))
    oc = torch.from_numpy(w.outlier_ch) if w.outlier_ch is not None else None
    base = KvcCache(w.fmt, w.batch, w.hkv, cap, page_size=w.page_size, block_table=table,
                    num_pages=num_pages, fp16_rows=w.fp16_shadow, kT=w.kT, outlier_ch=oc,
                    outlier_v=w.outlier_v)
    base.append(torch.from_numpy(w.k).to(dev), torch.from_numpy(w.v).to(dev),
                torch.from_numpy(w.seq_lens).to(dev))
    torch.cuda.synchronize()
    nrep = max(1, math.ceil(args.replica_bytes / base.nbytes()))
    reps = [base] + [base.clone() for _ in range(nrep - 1)]
    return base, reps, cap


def replay_us(fns, calls: int) -> float:
    """Average duration of one call when `fns` (callables taking a stream, one
    call each) are captured in one HIP graph and replayed until at least
    `calls` calls have run, bracketed by events on the launch stream."""
    import torch
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for f in fns:
            f(st)
    torch.cuda.synchronize()
    g.replay()   # (warm)
    torch.cuda.synchronize()
    reps = -(-calls // len(fns))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(fns)) * 1e3


def attend_gate(name: str, args, calls: int) -> dict:
    """The kvc_attend_decode call alone on a dense workload (graph replay over
    rotated cache replicas): its duration and algorithmic HBM rate."""
    import numpy as np
    import torch
    import workloads as W
    from decode_attention_sparse_kvc_amd import kvc
    w = W.FULL[name]()
    base, reps, cap = make_caches(w, args, 64)
    dev = torch.device("cuda")
    q = torch.from_numpy(w.q).to(dev)
    out = torch.empty(w.batch, w.hq, 128, device=dev)
    lse = torch.empty(w.batch, w.hq, device=dev)
    nbytes = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, base.desc, w.hq, 0, 0, 0, 0, args.workgroups)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    per = len(reps) * -(-GRAPH_CALLS // len(reps))
    fns = [lambda st, r=i % len(reps): kvc.kvc_attend_decode(
        reps[r].desc, q, w.hq, w.sm_scale, 0, None, 0, 0, 0, out, lse, None, 0, ws, nbytes, st,
        workgroups=args.workgroups) for i in range(per)]
    us = replay_us(fns, calls)
    nb = attend_bytes(w, np.array(w.seq_lens, np.int64), None)
    achieved = nb / (us * 1e-6) / 1e9
    del reps, base
    torch.cuda.empty_cache()
    return {"workload": name, "launch_us": us, "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": nb,
            "context_tokens_per_s": float(np.sum(w.seq_lens)) / (us * 1e-6)}


def stream_ceiling(call_bytes: int, total_bytes: float, calls: int) -> dict:
    """Plain streaming read (kvc_stream_read) over a buffer of total_bytes:
    once per call over the whole buffer, and in call_bytes pieces rotating
    over it (the size of one attend call's reads, launch and ramp included)."""
    import torch
    from decode_attention_sparse_kvc_amd import kvc
    chunk = (int(call_bytes) + 4095) // 4096 * 4096
    nchunk = max(2, math.ceil(total_bytes / chunk))
    buf = torch.ones(nchunk * chunk, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4 * 1024, dtype=torch.int32, device="cuda")
    wg = 1024
    whole = replay_us([lambda st: kvc.kvc_stream_read(buf, buf.numel(), sink, wg, st)] * 4, 8)
    pieces = replay_us([lambda st, i=i: kvc.kvc_stream_read(buf[(i % nchunk) * chunk:], chunk, sink, wg, st)
                        for i in range(nchunk)], calls)
    res = {"kernel": "kvc_stream_read", "unit": "GB/s",
           "read_GBs_whole": buf.numel() / (whole * 1e-6) / 1e9, "whole_bytes": buf.numel(),
           "read_GBs_call_size": chunk / (pieces * 1e-6) / 1e9, "call_bytes": chunk,
           "call_size_us": pieces}
    del buf
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; the path shards by (sequence, KV head) "
              "with no exchange, so N-GPU throughput is N times the 1-GPU figure by construction "
              "and is not measured here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import workloads as W
    from decode_attention_sparse_kvc_amd import KvcCache, kvc

    w = W.FULL[args.workload]()
    dev = torch.device("cuda")
    extra = args.warmup + 2 * args.steps + 2 * GRAPH_CALLS + 64   # room for the tokens the steps append
    base, reps, cap = make_caches(w, args, extra)
    nrep = len(reps)
    lens = [np.array(w.seq_lens, np.int64) for _ in reps]

    q = torch.from_numpy(w.q).to(dev)
    k_new = torch.from_numpy(w.k_new).to(dev)
    v_new = torch.from_numpy(w.v_new).to(dev)
    mode = kvc.MODE[w.mode]
    sparse = w.score is not None
    k_max = int(w.top_k.max()) if sparse else 0
    out = torch.empty(w.batch, w.hq, 128, device=dev)
    lse = torch.empty(w.batch, w.hq, device=dev)
    nbytes = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, base.desc, w.hq, mode, k_max, w.n_sink, w.n_window,
                                     args.workgroups)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if sparse:
        tk_bytes = kvc.kvc_workspace_bytes(kvc.OP_SCORE_TOPK, base.desc, w.hq)
        tk_ws = torch.empty(tk_bytes, dtype=torch.uint8, device=dev)
        sel = torch.full((w.batch, w.hkv, k_max), -1, dtype=torch.int32, device=dev)
        k_per_seq = torch.from_numpy(w.top_k.astype(np.int32)).to(dev)
    accs = None
    if w.accumulate:
        acc0 = np.zeros((w.batch, w.hkv, cap), np.float32)
        acc0[:, :, : w.acc.shape[2]] = w.acc[:, :, :cap]
        accs = [torch.from_numpy(acc0).to(dev) for _ in reps]
        stride = (w.n_sink + k_max + w.n_window if w.mode == "drop"
                  else w.n_sink + 64 * k_max + w.n_window if w.mode == "blocks" else cap)
        logits = torch.empty(w.batch, w.hq, stride, device=dev)
    if w.prefer_k and not w.accumulate:   # the attention rows the top-k mass reads
        stride = cap
        logits = torch.empty(w.batch, w.hq, stride, device=dev)
    mass = torch.empty(w.batch, w.hq, device=dev)
    tm_bytes = kvc.kvc_workspace_bytes(kvc.OP_TOPK_MASS, base.desc, w.hq) if w.prefer_k else 0
    tm_ws = torch.empty(max(tm_bytes, 16), dtype=torch.uint8, device=dev)
    want_logits = bool(accs) or w.prefer_k > 0
    names = (["append"] + (["score_topk"] if sparse else []) + ["attend"] + (["accum"] if accs else [])
             + (["topk_mass"] if w.prefer_k else []))

    def op_append(r, st):
        kvc.kvc_quantize_append(reps[r].desc, k_new, v_new, None, 1, None, st)

    score_mode = (kvc.SCORE[w.score] | (kvc.SCORE_BLOCKS if w.granule == "block" else 0)) if sparse else 0

    def op_score_topk(r, st):
        ext = accs[r] if w.score == "external" else None
        kvc.kvc_score_topk(reps[r].desc, q, w.hq, score_mode, w.n_crit, ext, w.n_sink,
                           w.n_window, k_per_seq, k_max, sel, None, None, tk_ws, tk_bytes, st)

    def op_attend(r, st):
        kvc.kvc_attend_decode(reps[r].desc, q, w.hq, w.sm_scale, mode, sel if sparse else None,
                              k_max, w.n_sink, w.n_window, out, lse, logits if want_logits else None,
                              stride if want_logits else 0, ws, nbytes, st, workgroups=args.workgroups)

    def op_accum(r, st):
        kvc.kvc_accum_scores(reps[r].desc, w.hq, logits, stride, lse, mode, sel if sparse else None,
                             k_max, w.n_sink, w.n_window, accs[r], st)

    def op_topk_mass(r, st):
        kvc.kvc_topk_mass(reps[r].desc, w.hq, logits, stride, lse, w.prefer_k, mass, tm_ws, tm_bytes,
                          st)

    ops = {"append": op_append, "score_topk": op_score_topk, "attend": op_attend, "accum": op_accum,
           "topk_mass": op_topk_mass}

    def step(r, st):
        for nm in names:
            ops[nm](r, st)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i % nrep, stream)
        lens[i % nrep] += 1
    torch.cuda.synchronize()

    def capture(fn):
        """A HIP graph of fn(stream); nothing runs until it is replayed."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(torch.cuda.current_stream())
        return g

    # The timed steps, replicas in rotation: step s uses replica (warmup + s) % nrep.
    order = [(args.warmup + s_) % nrep for s_ in range(args.steps)]
    graph = not args.no_graph
    # a replayed graph holds whole passes over the replicas, at least
    # GRAPH_CALLS steps (as one graph would hold every layer of a model's
    # decode step), so the graph launch is amortized as it would be there;
    # a remainder of fewer steps replays single-step graphs
    per = nrep * -(-GRAPH_CALLS // nrep)
    if graph:
        rounds = args.steps // per
        seq = order[:per]
        pass_graph = capture(lambda st: [step(r, st) for r in seq]) if rounds else None
        tail_graphs = {r: capture(lambda st, r=r: step(r, st)) for r in order[rounds * per:]}
        torch.cuda.synchronize()

    # host bookkeeping of the timed steps, done before the timed region
    ctx_tokens = 0
    for r in order:
        lens[r] += 1
        ctx_tokens += int(lens[r].sum())

    # ---- timed region: exactly `steps` steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    if graph:
        for _ in range(rounds):
            pass_graph.replay()
        for r in order[rounds * per:]:
            tail_graphs[r].replay()
    else:
        for r in order:
            step(r, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # ---- per-op durations: each op alone, `per` calls per graph (whole passes
    # over the replicas), replayed until at least `steps` calls have run,
    # bracketed by events on the launch stream
    per_op_us = {}
    for nm in names:
        if graph:
            g = capture(lambda st: [ops[nm](i % nrep, st) for i in range(per)])
            torch.cuda.synchronize()
        reps_needed = -(-args.steps // per)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps_needed):
            if graph:
                g.replay()
            else:
                for i in range(per):
                    ops[nm](i % nrep, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_op_us[nm] = e0.elapsed_time(e1) / (reps_needed * per) * 1e3
        if nm == "append":
            for r in range(nrep):
                lens[r] += reps_needed * (per // nrep)
    attend_us = per_op_us["attend"]
    attend_calls_bytes = sum(attend_bytes(w, lens[r], w.top_k if sparse else None)
                             for r in range(nrep)) / nrep
    achieved = attend_calls_bytes / (attend_us * 1e-6) / 1e9
    digest = src_digest()
    traffic = read_traffic("attend_kernel", args.workload, digest)
    step_desc = " + ".join({"append": "kvc_quantize_append(1 token)",
                            "score_topk": f"kvc_score_topk({w.score})",
                            "attend": f"kvc_attend_decode({w.mode})",
                            "accum": "kvc_accum_scores",
                            "topk_mass": f"kvc_topk_mass(k={w.prefer_k})"}[nm] for nm in names)

    result = {
        "metric": "decode attention context-tokens/s per layer at 128K; achieved HBM GB/s vs peak",
        "value": ctx_tokens / (total_ms * 1e-3),
        "unit": "context-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "format": w.fmt,
            "batch": w.batch,
            "context": int(w.seq_lens.max()),
            "context_total": int(w.seq_lens.sum()),
            "q_heads": w.hq,
            "kv_heads": w.hkv,
            "head_dim": 128,
            "step": step_desc,
            "cache_replicas": nrep,
            "replica_bytes": base.nbytes(),
            "per_op_us": per_op_us,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kvc_attend_decode call (attend_kernel + merge_kernel)",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": attend_calls_bytes,
            "launch_us": attend_us,
            "src_digest": digest,
        },
    }
    calls = max(args.steps, 2 * GRAPH_CALLS)
    if not args.no_ceiling:
        ceil = stream_ceiling(attend_calls_bytes, args.replica_bytes, calls)
        result["roofline"]["ceiling"] = ceil
        result["roofline"]["frac_of_ceiling"] = achieved / ceil["read_GBs_whole"]
    if args.workload == DEFAULT_WORKLOAD and not args.no_gates:
        # both gated calls of the layer at 128K: this INT4 layer's (above) and
        # the 1-bit layer's, measured the same way in the same run
        result["roofline"]["gates"] = {
            "int4_128k": {"workload": args.workload, "launch_us": attend_us, "achieved": achieved,
                          "frac": achieved / PEAK_HBM_GBS},
            "int1_128k": attend_gate("llama8b_layer_int1_dense_128k", args, calls),
        }
    if not args.no_cpu_baseline:
        if w.mode == "dense":
            result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_seconds)
        else:
            result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
