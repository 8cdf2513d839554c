"""Run a synthetic serving script through the oracle.

Test infrastructure only (see `oracle/__init__.py`).

The pool starts with a NaN canary in every slot (stale memory).  Each step
runs the block manager over its operations, applies the copy-on-write block
copies it asked for, then writes the step's K/V rows through the slots it
returned (copies first: a copy takes the block as it was before this step's
writes).  Rows of prompt tokens found in the prefix cache are not written:
their K/V is already in the pool ("vLLM" page, Prefix Caching: a hit skips
prefill).  After the final step, the measured batch is attended.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from . import attention
from .block_manager import OracleBlockManager

_CANARY = {"bf16": (np.uint16, 0x7FC1), "f32": (np.uint32, 0x7FC00001), "fp8": (np.uint8, 0x7F)}


def kv_dtype(w) -> str:
    """Element type of the caches: the workload's dtype, or "fp8" (E4M3
    codes with per-KV-head scales w.k_scale, w.v_scale) when w.kv_dtype says so."""
    return getattr(w, "kv_dtype", None) or w.dtype


@dataclasses.dataclass
class OracleState:
    bm: OracleBlockManager
    k_cache: np.ndarray
    v_cache: np.ndarray
    step_slots: List[np.ndarray]                # per step, int32 slot of each appended token
    step_copies: List[List[Tuple[int, int]]]    # per step, (src, dst) copies
    block_tables: np.ndarray                    # [batch][max_blocks] int32, -1 padded
    context_lens: np.ndarray                    # [batch] tokens after the final step
    query_start_loc: np.ndarray                 # [batch+1] rows of the final step's tokens
    prefill_skipped: int = 0                    # prompt tokens served by the prefix cache


def new_pool(w):
    """Pool of canary-filled K and V caches [num_blocks][B][H_kv][D]."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    ut, bits = _CANARY[kv_dtype(w)]
    kc = np.full(shape, bits, dtype=ut)
    vc = np.full(shape, bits, dtype=ut)
    if kv_dtype(w) == "f32":
        kc, vc = kc.view(np.float32), vc.view(np.float32)
    return kc, vc


def run_script(w, max_blocks: Optional[int] = None) -> OracleState:
    bm = OracleBlockManager(w.num_blocks, w.block_size, w.free_order)
    kc, vc = new_pool(w)
    slots_all, copies_all = [], []
    skipped = 0
    for step in list(w.history) + [w.final]:
        rows = []
        slots, copies = bm.apply(step.ops, rows)
        attention.copy_blocks(kc, vc, copies)
        k, v = step.k[rows], step.v[rows]
        skipped += len(step.k) - len(rows)
        if kv_dtype(w) == "fp8":
            attention.cache_write_fp8(k, v, slots, kc, vc, w.k_scale, w.v_scale)
        else:
            attention.cache_write(k, v, slots, kc, vc)
        slots_all.append(np.asarray(slots, dtype=np.int32))
        copies_all.append(copies)
    batch = [int(s) for s in w.batch]
    need = max([len(bm.tables[s]) for s in batch] + [1])
    width = need if max_blocks is None else max_blocks
    tables = np.full((len(batch), width), -1, dtype=np.int32)
    for r, s in enumerate(batch):
        t = bm.tables[s]
        tables[r, : len(t)] = t
    lens = np.asarray([bm.num_tokens[s] for s in batch], dtype=np.int32)
    qlen = {s: 0 for s in batch}
    for op in w.final.ops:
        if op[0] == "prompt":
            raise ValueError("the measured step appends tokens; prompts arrive before it")
        if op[0] == "append":
            qlen[op[1]] += op[2]
    qsl = np.zeros(len(batch) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([qlen[s] for s in batch])
    return OracleState(bm, kc, vc, slots_all, copies_all, tables, lens, qsl, skipped)


def attend(w, st: OracleState, pairs=None) -> np.ndarray:
    """The final step's attention output, float64 (all outputs, or `pairs`)."""
    kv = {}
    if kv_dtype(w) != w.dtype:
        kv = dict(cache_dtype=kv_dtype(w), k_scale=w.k_scale, v_scale=w.v_scale)
    if w.kind == "decode":
        return attention.decode(w.q, st.k_cache, st.v_cache, st.block_tables,
                                st.context_lens, w.scale, w.dtype, w.num_kv_heads, pairs, **kv)
    return attention.varlen(w.q, st.query_start_loc, st.context_lens, st.k_cache,
                            st.v_cache, st.block_tables, w.scale, w.dtype,
                            w.num_kv_heads, pairs, **kv)
