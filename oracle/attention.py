"""Oracle cache write, block-table gather and attention, in float64.

Test infrastructure only (see `oracle/__init__.py`).

What the pages fix, and where:

* Each new token's K/V is stored in the slot the model runner computed for
  it (slot_mapping), and the attention kernel finds a request's data in the
  physical blocks through the same mapping (CSDN "vLLM 0.10.0" page, §3.3
  steps 4–5 and §4 step 4).
* The attention operator receives Q as the flattened tokens of the batch,
  KV as the whole per-layer cache tensor, and metadata: block table,
  slot_mapping and query_start_loc separating requests (same page, §3.5).
* Decode reads the request's logical blocks as if contiguous while the data
  is fetched from physical blocks through the block table (SourceAIX page
  §5.1.1 step (2); "vLLM" page, section "PagedAttention 的解决方案").  The
  result is therefore plain softmax attention over the request's logical
  KV sequence.
* A token attends only to itself and earlier tokens (causal mask; dn008
  page, §2.1), which is what a chunked-prefill row obeys
  (CSDN page §3.2, chunked prefill mixed with decode).
* GQA: several query heads share one KV head (CSDN page §3.4; "vLLM" page,
  tuning section).
* An "fp8" cache holds E4M3 codes with one scale per KV head (fp8.py, an
  extension: the pages name 8-bit floats for weights only); attention sees
  each code times its scale.
* A preempted group's KV blocks are swapped out to CPU memory and later
  swapped back in, after which its inference continues (SourceAIX page
  §6.2.1, steps (3)–(4)): a block move keeps the block's contents, so the
  request's attention is unchanged once its table names the new blocks.

Readings (listed in the design doc): the cache tensor is
[num_blocks][block_size][num_kv_heads][head_dim], so a slot is one row of
its [num_blocks*block_size][num_kv_heads][head_dim] view; query head h uses
KV head h // (num_heads / num_kv_heads); a negative slot means "no write";
a request with no token attends to nothing and outputs zeros.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import fp8


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements.

    A bfloat16 value is the float32 whose upper 16 bits are the stored bits
    and whose lower 16 bits are zero.
    """
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def cache_write(k, v, slot_mapping, k_cache, v_cache) -> None:
    """k_cache[slot] = k[i], v_cache[slot] = v[i] for every token i with slot >= 0.

    Exact element copies; every other slot is left as it was.
    """
    nb, bs, hkv, d = k_cache.shape
    kc = k_cache.reshape(nb * bs, hkv, d)
    vc = v_cache.reshape(nb * bs, hkv, d)
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        kc[slot] = k[i]
        vc[slot] = v[i]


def cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale) -> None:
    """cache_write into E4M3 caches (uint8 codes): KV head h of token i is
    stored as the code of k[i][h] / k_scale[h] (same for v), see fp8.py.
    k, v: stored bf16 bits [T][H_kv][D]; scales: float32 [H_kv]."""
    nb, bs, hkv, d = k_cache.shape
    kc = k_cache.reshape(nb * bs, hkv, d)
    vc = v_cache.reshape(nb * bs, hkv, d)
    kf, vf = to_f64(k, "bf16"), to_f64(v, "bf16")
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        for h in range(hkv):
            kc[slot, h] = fp8.quantize(kf[i, h], np.float32(k_scale[h]))
            vc[slot, h] = fp8.quantize(vf[i, h], np.float32(v_scale[h]))


def copy_blocks(k_cache, v_cache, copies: Iterable[Tuple[int, int]]) -> None:
    """Copy-on-write block copies: the whole block src → dst, K and V."""
    for src, dst in copies:
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(src_k, src_v, dst_k, dst_v, moves: Iterable[Tuple[int, int]]) -> None:
    """Swap out / swap in (SourceAIX page §6.2.1): the whole block src of one
    pool (e.g. the GPU caches) becomes block dst of another (e.g. a CPU pool),
    K and V; blocks keep their slot layout, so a later move back restores the
    pool exactly."""
    for src, dst in moves:
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def logical_rows(block_table: Sequence[int], length: int, block_size: int) -> List[int]:
    """Row (slot) index of each logical token 0..length-1 through the table."""
    return [int(block_table[t // block_size]) * block_size + t % block_size
            for t in range(length)]


def gather(cache, block_table, length: int, dtype: str, scale=None) -> np.ndarray:
    """The request's logical K (or V) rows [length][num_kv_heads][head_dim] in
    float64; for an "fp8" cache each code times its KV head's scale."""
    nb, bs, hkv, d = cache.shape
    flat = cache.reshape(nb * bs, hkv, d)
    rows = logical_rows(block_table, length, bs)
    if not rows:
        return np.zeros((0, hkv, d))
    if dtype == "fp8":
        sc = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return fp8.decode(flat[np.asarray(rows)]) * sc[None, :, None]
    return to_f64(flat[np.asarray(rows)], dtype)


def _attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K qv) weighted sum of V rows; zeros over an empty K."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ qv)
    z = z - z.max()
    p = np.exp(z)
    p = p / p.sum()
    return p @ V


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
           num_kv_heads: int, pairs: Optional[Iterable[Tuple[int, int]]] = None,
           cache_dtype: Optional[str] = None, k_scale=None, v_scale=None) -> np.ndarray:
    """One query row per sequence over its context_lens[s] logical tokens.

    q: [num_seqs][H][D] stored values.  Returns float64 [num_seqs][H][D];
    with `pairs` only those (seq, head) outputs are computed (others NaN).
    The caches hold `cache_dtype` (default: dtype); "fp8" caches are
    dequantised with the per-KV-head scales.
    """
    cd = cache_dtype or dtype
    n, H, D = q.shape
    G = H // num_kv_heads
    out = np.full((n, H, D), np.nan) if pairs is not None else np.zeros((n, H, D))
    want = None if pairs is None else {}
    if pairs is not None:
        for s, h in pairs:
            want.setdefault(int(s), []).append(int(h))
    qf = to_f64(q, dtype)
    for s in range(n):
        heads = range(H) if want is None else want.get(s, [])
        if not heads:
            continue
        L = int(context_lens[s])
        K = gather(k_cache, block_tables[s], L, cd, k_scale)
        V = gather(v_cache, block_tables[s], L, cd, v_scale)
        for h in heads:
            g = h // G
            out[s, h] = _attend(qf[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def varlen(q, query_start_loc, seq_lens, k_cache, v_cache, block_tables, scale: float,
           dtype: str, num_kv_heads: int,
           rows: Optional[Iterable[Tuple[int, int]]] = None,
           cache_dtype: Optional[str] = None, k_scale=None, v_scale=None) -> np.ndarray:
    """Chunked prefill and decode rows in one batch.

    Sequence s owns query rows [qsl[s], qsl[s+1]); with q_len of them and
    L = seq_lens[s] tokens in total, the row at index i of the segment is
    the token at position L - q_len + i and attends to keys 0 .. L-q_len+i.
    Returns float64 [total_q][H][D]; with `rows` only those (row, head)
    outputs are computed (others NaN).
    """
    T, H, D = q.shape
    G = H // num_kv_heads
    out = np.full((T, H, D), np.nan) if rows is not None else np.zeros((T, H, D))
    want = None
    if rows is not None:
        want = {}
        for r, h in rows:
            want.setdefault(int(r), []).append(int(h))
    qf = to_f64(q, dtype)
    cd = cache_dtype or dtype
    n = len(seq_lens)
    for s in range(n):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        if b <= a:
            continue
        if want is not None and not any(r in want for r in range(a, b)):
            continue
        L = int(seq_lens[s])
        prior = L - (b - a)
        K = gather(k_cache, block_tables[s], L, cd, k_scale)
        V = gather(v_cache, block_tables[s], L, cd, v_scale)
        for i in range(b - a):
            r = a + i
            heads = range(H) if want is None else want.get(r, [])
            last = prior + i  # position of this row's token; keys 0..last
            for h in heads:
                g = h // G
                out[r, h] = _attend(qf[r, h], K[: last + 1, g, :], V[: last + 1, g, :], scale)
    return out
