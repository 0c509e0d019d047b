"""CPU oracle for one decode step of attention over a jointly sparsified + quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or constant generator with the HIP library under
``decode_attention_sparse_kvc_amd/``; both sides read the same seeded inputs
from ``workloads`` and nothing else.

It is written to be read against the pages, not to be fast: numpy, fp32 where
the quantizer's own arithmetic is the specification, fp64 everywhere else, one
plain step at a time in the pages' order.

  quant   -- asymmetric min-max quantizer (TailorKV article, section 2.2, the
             printed ``quant_1bit`` generalized by its own 2**b - 1 levels);
             K per channel over 64-token groups, V per token over 64-channel
             groups (same section; on-device KV article, section 3.1);
             outlier channels (K, optionally V) kept at fp16 beside the codes, chosen by
             variance (meeting-LLM article, section 8.2).
  select  -- critical channels and approximate scores (TailorKV, section 2.3),
             exact query-aware scores, Top-K with lower-index ties, sinks and
             recent window (StreamingLLM / H2O survey, section 3).
  attend  -- softmax(q K^T / sqrt(d)) V over the attended set with GQA (TailorKV
             section 2.1's attention definition; FlashDecoding-Sparse sketch in
             the meeting-LLM article, section 8.1, for what one decode step
             computes), lse, logits, and the H2O cumulative-score update
             (StreamingLLM / H2O survey, section 3.2).
  step    -- the pipeline of one decode step per workload, built from the above.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, worked examples, brute force and textbook routines.  Parity
unpinned: none of the functions; the pages' quality numbers (accuracy, PPL)
are out of reach without models and are not claimed.
"""
