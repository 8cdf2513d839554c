"""CPU oracle for the paged KV-cache attention path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct reference code, written from the pages'
description of PagedAttention (vLLM):

* `block_manager`  — the logical→physical block mapping with on-demand
  allocation, per-block reference counts and copy-on-write
  ("vLLM" documentation page, sections "算法流程", "引用计数管理", "写时复制";
  SourceAIX "PagedAttention算法" §5.1.1 and §5.2.1).
* `attention`      — the slot_mapping scatter into the cache, the gather of a
  request's logical KV through its block table, and softmax attention over
  it in float64 (decode rows and causal chunked-prefill rows).
* `run`            — applies a synthetic serving script to both.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import this package.  It shares no code with the HIP path and
imports nothing from it; the product never calls it.

Parity status: every function here is pinned by `tests/test_oracle_*.py`
against the pages' worked examples, closed forms, invariants and library
routines (see the module headers); none is "parity unpinned".
"""
