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

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: this build runs on
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
CODE_BYTES = {"int4": 144, "int1": 48}      # per token per KV head, incl. amortized K meta


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--replica-bytes", type=float, default=1.5 * 2**30,
                    help="total bytes of rotated cache replicas (defeats the Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def src_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_sparse_kvc_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
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


def attend_bytes(fmt: str, lens, hkv: int, hq: int, batch: int) -> int:
    """Algorithmic bytes of one kvc_attend_decode over every cached token (dense)."""
    total = 0
    for n in lens:
        nq = (int(n) // 64) * 64
        per_head = nq * CODE_BYTES[fmt] + (int(n) - nq) * 512 if fmt != "fp16" else int(n) * 512
        total += hkv * per_head
    total += batch * hq * 128 * 2           # q
    total += batch * hq * (128 + 1) * 4     # out + lse
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


def cpu_baseline(w, seconds: float):
    """The oracle's decode step on a bounded sample: whole KV heads, timed on host cores."""
    from threadpoolctl import threadpool_limits
    from oracle import step as ST
    pairs_all = [(b, g) for b in range(w.batch) for g in range(w.hkv)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        done = []
        for p in pairs_all:
            ST.decode_step(w, append=True, pairs=[p])
            done.append(p)
            if time.perf_counter() - t0 > seconds:
                break
        dt = time.perf_counter() - t0
    frac = len(done) / len(pairs_all)
    ctx = sum(int(w.seq_lens[b]) + 1 for b in range(w.batch))
    return {
        "value": ctx * frac / dt,
        "unit": "context-tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(done)} of {len(pairs_all)} (sequence, KV head) pairs, each a full "
                  f"decode step (append + quantize + attend over the whole context) in numpy "
                  f"on 1 thread, {dt:.1f} s; scaled by the fraction of pairs",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; the path shards by (sequence, KV head) "
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
    if w.mode != "dense":
        raise SystemExit(f"bench.py: workload {args.workload} needs kvc_score_topk (not built yet)")
    dev = torch.device("cuda")
    table = torch.from_numpy(w.block_table) if w.block_table is not None else None
    extra = args.warmup + args.steps + 64
    cap = ((int(w.seq_lens.max()) + extra + 63) // 64) * 64
    base = KvcCache(w.fmt, w.batch, w.hkv, cap, page_size=w.page_size, block_table=table,
                    num_pages=w.num_pages, fp16_rows=w.fp16_shadow, kT=w.kT)
    base.append(torch.from_numpy(w.k).to(dev), torch.from_numpy(w.v).to(dev),
                torch.from_numpy(w.seq_lens).to(dev))
    torch.cuda.synchronize()
    nrep = max(1, math.ceil(args.replica_bytes / base.nbytes()))
    reps = [base] + [base.clone() for _ in range(nrep - 1)]
    lens = [np.array(w.seq_lens, np.int64) for _ in reps]

    q = torch.from_numpy(w.q).to(dev)
    k_new = torch.from_numpy(w.k_new).to(dev)
    v_new = torch.from_numpy(w.v_new).to(dev)
    mode = kvc.MODE[w.mode]
    out = torch.empty(w.batch, w.hq, 128, device=dev)
    lse = torch.empty(w.batch, w.hq, device=dev)
    nbytes = kvc.kvc_workspace_bytes(kvc.OP_ATTEND, base.desc, w.hq, mode, 0, 0, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        r = i % nrep
        c = reps[r]
        kvc.kvc_quantize_append(c.desc, k_new, v_new, None, 1, None, stream)
        lens[r] += 1
        if ev is not None:
            ev[0].record(stream)
        kvc.kvc_attend_decode(c.desc, q, w.hq, w.sm_scale, mode, None, 0, 0, 0, out, lse,
                              None, 0, ws, nbytes, stream)
        if ev is not None:
            ev[1].record(stream)
        return r

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    ctx_tokens = 0
    att_bytes = 0
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        r = step(args.warmup + s, events[s])
        ctx_tokens += int(lens[r].sum())
        att_bytes += attend_bytes(w.fmt, lens[r], w.hkv, w.hq, w.batch)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    attend_ms = sum(a.elapsed_time(b) for a, b in events)
    ms_per_step = total_ms / args.steps
    attend_us = attend_ms / args.steps * 1e3
    achieved = att_bytes / args.steps / (attend_us * 1e-6) / 1e9
    digest = src_digest()
    traffic = read_traffic("attend_kernel", args.workload, digest)

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
            "q_heads": w.hq,
            "kv_heads": w.hkv,
            "head_dim": 128,
            "step": "kvc_quantize_append(1 token) + kvc_attend_decode(dense)",
            "cache_replicas": nrep,
            "replica_bytes": base.nbytes(),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kvc_attend_decode (attend_kernel + split merge)",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": att_bytes / args.steps,
            "launch_us": attend_us,
            "src_digest": digest,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
