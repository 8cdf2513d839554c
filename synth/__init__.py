"""Seeded synthetic workloads for the paged KV-cache attention path.

This module only *draws inputs*: sequence lengths, the order in which the
physical block pool hands out blocks, the operation script a serving engine
would issue (new sequence, fork, append tokens, free), the K/V rows of every
appended token and the query rows of the final step.  It contains none of the
method's arithmetic: no block allocation, no slot computation, no attention.
Both the CPU oracle and the HIP path consume the same `Workload` and each
derives block tables, slot mappings and outputs on its own.

Values are drawn in float32 from NumPy's PCG64 (`default_rng(seed)`), and for
bf16 workloads rounded to bfloat16 bit patterns (round to nearest, ties to
even) here, so that both sides receive identical bits.

The five named workloads follow the shapes of the pages' problem statement
(a fixed-size block KV cache reached through per-request block tables, the
16-token default block and the 4-token worked example, GQA head grouping,
parallel-sampling prefix sharing, chunked prefill mixed with decode).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# bf16 bit patterns (input preparation only)
# ---------------------------------------------------------------------------

# Quiet-NaN canary written into every slot that no token ever owns, so a
# kernel that reads a stale slot, or multiplies a masked V row by zero,
# shows up as NaN.
CANARY_BF16 = np.uint16(0x7FC1)
CANARY_F32_BITS = np.uint32(0x7FC00001)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite draws from N(0,1); NaN/Inf are not expected.
    Works in chunks so that large pools do not need several full-size
    temporaries.
    """
    src = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(src.shape, dtype=np.uint16)
    step = 1 << 22
    for a in range(0, src.size, step):
        u = src[a:a + step].copy()
        lsb = u >> np.uint32(16)
        lsb &= np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u >>= np.uint32(16)
        out[a:a + step] = u
    return out.reshape(np.shape(x))


# ---------------------------------------------------------------------------
# Workload description
# ---------------------------------------------------------------------------

# An operation of the serving script, applied in list order:
#   ("new", sid)            a request arrives with an empty block table
#   ("fork", parent, child) child starts as a copy of parent's logical view
#                           (parallel sampling: the same prompt, shared blocks)
#   ("append", sid, n)      n tokens of sid get K/V (prefill chunk or decode)
#   ("prompt", sid, tokens) a request arrives with its prompt's token ids
#                           (a tuple); the step carries K/V rows for every
#                           prompt token, and the consumer writes only those
#                           its prefix cache does not already hold
#   ("free", sid)           the request finished
Op = Tuple


@dataclasses.dataclass
class Step:
    ops: List[Op]
    k: np.ndarray  # [n_appended][H_kv][D] storage dtype (uint16 bf16 bits or float32)
    v: np.ndarray


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                 # "decode" or "varlen"
    dtype: str                # "bf16" or "f32"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray    # int32 permutation of [0, num_blocks): pool hand-out order
    history: List[Step]       # steps before the measured one (cache fill, untimed)
    final: Step               # the measured step: its tokens are written, then attended
    batch: np.ndarray         # int32 sequence ids forming the batch rows, in order
    q: np.ndarray             # decode: [len(batch)][H][D]; varlen: [total_q][H][D]
    scale: float
    partition_size: int = 0   # 0: library default
    notes: str = ""
    kv_dtype: Optional[str] = None         # "fp8": caches of E4M3 codes (q, k, v stay in dtype)
    k_scale: Optional[np.ndarray] = None   # fp8: float32 [H_kv] scale of each KV head's codes
    v_scale: Optional[np.ndarray] = None

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def cache_elem_bytes(self) -> int:
        """Bytes of one cache element (1 for E4M3 caches)."""
        return 1 if self.kv_dtype == "fp8" else self.elem_bytes

    def final_appends(self) -> List[Tuple[int, int]]:
        """(sid, n) of every append in the final step, in order."""
        return [(op[1], op[2]) for op in self.final.ops if op[0] == "append"]


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _store(rng.standard_normal(shape, dtype=np.float32), dtype)


def _free_order(seed: int, num_blocks: int) -> np.ndarray:
    return np.random.default_rng(seed + 1).permutation(num_blocks).astype(np.int32)


def _step(rng, ops, n_tokens, hkv, d, dtype) -> Step:
    return Step(ops=ops, k=_draw(rng, (n_tokens, hkv, d), dtype),
                v=_draw(rng, (n_tokens, hkv, d), dtype))


# ---------------------------------------------------------------------------
# Generic builders
# ---------------------------------------------------------------------------

def decode_workload(name, ctx_lens, *, num_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, dtype, seed, partition_size=0,
                    free_order=None, notes="") -> Workload:
    """Independent sequences; sequence i holds ctx_lens[i] tokens after the step.

    History: every sequence is created and its first ctx-1 tokens appended
    (one prefill step).  Final step: one decode token per sequence (only
    sequences with ctx >= 1 take part; a 0-length row stays empty).
    """
    rng = np.random.default_rng(seed)
    ctx_lens = [int(c) for c in ctx_lens]
    n = len(ctx_lens)
    ops = [("new", i) for i in range(n)]
    n_hist = 0
    for i, c in enumerate(ctx_lens):
        if c > 1:
            ops.append(("append", i, c - 1))
            n_hist += c - 1
    hist = [_step(rng, ops, n_hist, num_kv_heads, head_dim, dtype)]
    fops = [("append", i, 1) for i, c in enumerate(ctx_lens) if c >= 1]
    final = _step(rng, fops, len(fops), num_kv_heads, head_dim, dtype)
    q = _draw(rng, (n, num_heads, head_dim), dtype)
    fo = _free_order(seed, num_blocks) if free_order is None else np.asarray(free_order, np.int32)
    return Workload(name=name, kind="decode", dtype=dtype, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, free_order=fo, history=hist, final=final,
                    batch=np.arange(n, dtype=np.int32), q=q,
                    scale=1.0 / math.sqrt(head_dim), partition_size=partition_size,
                    notes=notes)


def sampling_workload(name, *, groups, members, prefix_len, suffix_lens,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      dtype, seed, partition_size=0, notes="") -> Workload:
    """Parallel sampling: each group's prompt is prefilled once, then forked.

    Sequence id = group*members + member.  History: for every group the
    leader (member 0) is created and its prompt of prefix_len tokens
    appended, then members 1.. are forked from it (they share every prompt
    block).  A second history step appends suffix_len-1 private tokens to
    each member in ascending id order.  The final step appends one token
    per member.  suffix_lens[sid] counts the final token.
    """
    rng = np.random.default_rng(seed)
    n = groups * members
    ops = []
    for g in range(groups):
        lead = g * members
        ops.append(("new", lead))
        ops.append(("append", lead, prefix_len))
        for m in range(1, members):
            ops.append(("fork", lead, lead + m))
    h0 = _step(rng, ops, groups * prefix_len, num_kv_heads, head_dim, dtype)
    ops2, n2 = [], 0
    for sid in range(n):
        if suffix_lens[sid] > 1:
            ops2.append(("append", sid, int(suffix_lens[sid]) - 1))
            n2 += int(suffix_lens[sid]) - 1
    h1 = _step(rng, ops2, n2, num_kv_heads, head_dim, dtype)
    final = _step(rng, [("append", sid, 1) for sid in range(n)], n, num_kv_heads, head_dim, dtype)
    q = _draw(rng, (n, num_heads, head_dim), dtype)
    return Workload(name=name, kind="decode", dtype=dtype, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, free_order=_free_order(seed, num_blocks),
                    history=[h0, h1], final=final, batch=np.arange(n, dtype=np.int32),
                    q=q, scale=1.0 / math.sqrt(head_dim), partition_size=partition_size,
                    notes=notes)


def beam_search_workload(name, *, width, prompt_len, steps, num_heads, num_kv_heads,
                         head_dim, block_size, num_blocks, dtype, seed) -> Workload:
    """Beam search over the paged cache (SourceAIX page §5.2.2).

    Sequence 0 gets the prompt, then width-1 forks share it.  At each of the
    `steps` decoding steps the next beams are `width` continuations of the
    current ones: a seeded draw picks each continuation's parent (sorted,
    with repetition), a parent's first continuation keeps its id, every
    further one is a fork under a new id, and the beams nobody continues are
    freed (forks first, so blocks still shared stay allocated).  Then every
    beam appends one token.  Which beams survive is the search's business
    (token probabilities); here it is a seeded draw.  The last step is the
    measured one; the batch is its beams in ascending id order.
    """
    rng = np.random.default_rng(seed)
    ops = [("new", 0), ("append", 0, prompt_len)] + [("fork", 0, b) for b in range(1, width)]
    hist = [_step(rng, ops, prompt_len, num_kv_heads, head_dim, dtype)]
    beams = list(range(width))
    next_id = width
    final = None
    for t in range(steps):
        parents = sorted(int(p) for p in rng.choice(beams, size=width, replace=True))
        ops, new_beams, seen = [], [], set()
        for p in parents:
            if p not in seen:
                seen.add(p)
                new_beams.append(p)
            else:
                ops.append(("fork", p, next_id))
                new_beams.append(next_id)
                next_id += 1
        ops += [("free", b) for b in beams if b not in seen]
        beams = sorted(new_beams)
        ops += [("append", b, 1) for b in beams]
        st = _step(rng, ops, len(beams), num_kv_heads, head_dim, dtype)
        if t + 1 < steps:
            hist.append(st)
        else:
            final = st
    q = _draw(rng, (len(beams), num_heads, head_dim), dtype)
    return Workload(name=name, kind="decode", dtype=dtype, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, free_order=_free_order(seed, num_blocks),
                    history=hist, final=final, batch=np.asarray(beams, dtype=np.int32),
                    q=q, scale=1.0 / math.sqrt(head_dim))


def prefix_cache_workload(name, *, tenants, sys_len, user_lo, user_hi, arrivals, steps,
                          lifetime, gen_lo, gen_hi, num_heads, num_kv_heads, head_dim,
                          block_size, dtype, seed) -> Workload:
    """Multi-tenant serving with shared system prompts ("vLLM" page, Prefix
    Caching: requests of one tenant start with the same system prompt).

    Tenant t has a system prompt of sys_len token ids; each request's prompt
    is its tenant's system prompt followed by a user message of uniform
    [user_lo, user_hi] token ids that no other request uses.  At each of the
    `steps` history steps: the requests that arrived `lifetime` steps ago
    finish, every other live request appends uniform [gen_lo, gen_hi]
    generated tokens, and `arrivals` requests arrive with their prompts
    (tenant drawn with probability proportional to 1/(t+1)).  The final step
    appends one decode token to every live request; the batch is the live
    requests in ascending id order.

    The K/V rows of a system-prompt position are drawn once per tenant and
    repeated in every prompt of that tenant, so equal prefixes carry equal
    K/V (as a model's would); user and generated rows are fresh draws.  The
    pool holds exactly as many blocks as the live requests would need with
    no sharing at the busiest step, so blocks released with a cached prefix
    cycle to the front of the free list and get evicted.
    """
    rng = np.random.default_rng(seed)
    B = block_size
    vocab = 32000
    sys_tok = [tuple(int(x) for x in rng.integers(0, vocab, sys_len)) for _ in range(tenants)]
    sys_k = [_draw(rng, (sys_len, num_kv_heads, head_dim), dtype) for _ in range(tenants)]
    sys_v = [_draw(rng, (sys_len, num_kv_heads, head_dim), dtype) for _ in range(tenants)]
    pt = 1.0 / np.arange(1, tenants + 1)
    pt /= pt.sum()
    fresh = vocab                      # user token ids above the vocabulary: never shared
    live = {}                          # sid -> (arrival step, tokens held)
    hist, next_id, peak = [], 0, 0
    for t in range(steps):
        ops, ks, vs = [], [], []
        for sid in sorted(live):
            if live[sid][0] + lifetime == t:
                ops.append(("free", sid))
                del live[sid]
        for sid in sorted(live):
            g = int(rng.integers(gen_lo, gen_hi + 1))
            ops.append(("append", sid, g))
            ks.append(_draw(rng, (g, num_kv_heads, head_dim), dtype))
            vs.append(_draw(rng, (g, num_kv_heads, head_dim), dtype))
            live[sid] = (live[sid][0], live[sid][1] + g)
        for _ in range(arrivals):
            ten = int(rng.choice(tenants, p=pt))
            u = int(rng.integers(user_lo, user_hi + 1))
            toks = sys_tok[ten] + tuple(range(fresh, fresh + u))
            fresh += u
            ops.append(("prompt", next_id, toks))
            ks += [sys_k[ten], _draw(rng, (u, num_kv_heads, head_dim), dtype)]
            vs += [sys_v[ten], _draw(rng, (u, num_kv_heads, head_dim), dtype)]
            live[next_id] = (t, len(toks))
            next_id += 1
        hist.append(Step(ops=ops, k=np.concatenate(ks), v=np.concatenate(vs)))
        peak = max(peak, sum(-(-(n + (t == steps - 1)) // B) for _, n in live.values()))
    batch = sorted(live)
    final = _step(rng, [("append", sid, 1) for sid in batch], len(batch), num_kv_heads,
                  head_dim, dtype)
    q = _draw(rng, (len(batch), num_heads, head_dim), dtype)
    return Workload(name=name, kind="decode", dtype=dtype, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=B,
                    num_blocks=peak, free_order=_free_order(seed, peak), history=hist,
                    final=final, batch=np.asarray(batch, dtype=np.int32), q=q,
                    scale=1.0 / math.sqrt(head_dim))


def varlen_workload(name, segments, *, num_heads, num_kv_heads, head_dim,
                    block_size, num_blocks, dtype, seed, notes="") -> Workload:
    """Mixed chunked-prefill / decode step.

    segments: list of (prior, q_len).  Sequence i first holds `prior` tokens
    (history), then the final step appends q_len tokens whose queries form
    rows [query_start_loc[i], query_start_loc[i+1]) of q.  A decode row is
    q_len = 1.
    """
    rng = np.random.default_rng(seed)
    ops, n_hist = [], 0
    for i, (prior, _) in enumerate(segments):
        ops.append(("new", i))
        if prior > 0:
            ops.append(("append", i, int(prior)))
            n_hist += int(prior)
    hist = [_step(rng, ops, n_hist, num_kv_heads, head_dim, dtype)]
    fops = [("append", i, int(ql)) for i, (_, ql) in enumerate(segments) if ql > 0]
    total_q = sum(int(ql) for _, ql in segments)
    final = _step(rng, fops, total_q, num_kv_heads, head_dim, dtype)
    q = _draw(rng, (total_q, num_heads, head_dim), dtype)
    return Workload(name=name, kind="varlen", dtype=dtype, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, free_order=_free_order(seed, num_blocks),
                    history=hist, final=final,
                    batch=np.arange(len(segments), dtype=np.int32), q=q,
                    scale=1.0 / math.sqrt(head_dim), notes=notes)


# ---------------------------------------------------------------------------
# The five named workloads (full size) and their reduced twins
# ---------------------------------------------------------------------------

SEED_BASE = 1000


def tiny_f32(seed: int = SEED_BASE + 1) -> Workload:
    """2 sequences of 7 and 11 tokens, B=4, 4 heads = 4 KV heads, D=64, fp32,
    a 16-block pool handed out in a seeded random order; the step writes one
    new token per sequence (so 8 and 12 tokens are attended)."""
    return decode_workload("tiny_f32_decode", [8, 12], num_heads=4, num_kv_heads=4,
                           head_dim=64, block_size=4, num_blocks=16, dtype="f32",
                           seed=seed)


def gqa_decode(seed: int = SEED_BASE + 2, *, batch=32, lo=128, hi=2048,
               num_blocks=8192, partition_size=0) -> Workload:
    """bf16 GQA decode: 32 sequences, 32 query / 8 KV heads, D=128, B=16,
    context lengths uniform in [128, 2048] (counting the new token)."""
    rng = np.random.default_rng(seed + 7)
    ctx = rng.integers(lo, hi + 1, size=batch)
    return decode_workload("gqa_decode_b32", ctx, num_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, num_blocks=num_blocks,
                           dtype="bf16", seed=seed, partition_size=partition_size)


def long_context(seed: int = SEED_BASE + 3, *, batch=8, ctx=32768,
                 num_blocks=20480, partition_size=512) -> Workload:
    """bf16 long-context decode: 8 sequences of 32768 tokens, 64 query / 8 KV
    heads, D=128, B=16, 512-token split-K partitions."""
    return decode_workload("long_ctx_decode", [ctx] * batch, num_heads=64,
                           num_kv_heads=8, head_dim=128, block_size=16,
                           num_blocks=num_blocks, dtype="bf16", seed=seed,
                           partition_size=partition_size)


def parallel_sampling(seed: int = SEED_BASE + 4, *, groups=16, members=4,
                      prefix_len=1024, suffix_hi=256, num_blocks=4096) -> Workload:
    """bf16 parallel sampling: 16 groups of 4 sequences share a prompt of
    prefix_len tokens (ref_count 4), each with a private suffix of uniform
    [1, suffix_hi] tokens (counting the new one).  With a prompt that is not a
    multiple of B, the first write of each sharer into the partly filled last
    prompt block triggers copy-on-write."""
    rng = np.random.default_rng(seed + 7)
    suf = rng.integers(1, suffix_hi + 1, size=groups * members)
    return sampling_workload("parallel_sampling_cow", groups=groups, members=members,
                             prefix_len=prefix_len, suffix_lens=suf, num_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16,
                             num_blocks=num_blocks, dtype="bf16", seed=seed)


def parallel_sampling_unaligned(seed: int = SEED_BASE + 4, *, prefix_len=1020,
                                **kw) -> Workload:
    """The parallel-sampling workload with a 1020-token prompt: its last prompt
    block holds 12 of 16 slots, so the first write of three of the four
    sharers copies it (copy-on-write, 3 copies per group, 48 per step) and
    the fourth writes in place."""
    w = parallel_sampling(seed, prefix_len=prefix_len, **kw)
    w.name = "parallel_sampling_cow_1020"
    return w


def long_context_tp8_share(seed: int = SEED_BASE + 11, *, batch=8, ctx=32768,
                           num_blocks=20480, partition_size=0) -> Workload:
    """One GPU's share of the long-context decode under 8-way tensor
    parallelism by KV head: 8 sequences of 32768 tokens, 1 KV head and its
    8 query heads, D=128, B=16, bf16 (128 MiB of K/V per step).  The
    library's split choice (the balanced split): with one KV head, fixed
    512-token partitions would give only 512 waves."""
    return decode_workload("long_ctx_decode_tp8_share", [ctx] * batch, num_heads=8,
                           num_kv_heads=1, head_dim=128, block_size=16,
                           num_blocks=num_blocks, dtype="bf16", seed=seed,
                           partition_size=partition_size)


def mixed_varlen(seed: int = SEED_BASE + 5, *, n_prefill=4, chunk=512, prior_hi=3584,
                 n_decode=124, median=600.0, sigma=1.0, lo=16, hi=4096,
                 num_blocks=16384) -> Workload:
    """bf16 continuous-batching step: 4 chunked-prefill segments of 512 query
    tokens over a prior context uniform in [0, 3584], then 124 decode rows with
    log-normal context (median 600, natural-log sigma 1, rounded, clipped to
    [16, 4096], counting the new token)."""
    rng = np.random.default_rng(seed + 7)
    pri = rng.integers(0, prior_hi + 1, size=n_prefill)
    dec = np.clip(np.rint(rng.lognormal(math.log(median), sigma, size=n_decode)), lo, hi)
    segs = [(int(p), chunk) for p in pri] + [(int(c) - 1, 1) for c in dec]
    return varlen_workload("mixed_varlen", segs, num_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16, num_blocks=num_blocks,
                           dtype="bf16", seed=seed)


def mixed_varlen_prefill(seed: int = SEED_BASE + 5, **kw) -> Workload:
    """The four chunked-prefill segments of the bf16 continuous-batching step
    alone (same seed, so the same prior lengths and data draws), without its
    decode rows: the prefill part measured on its own."""
    w = mixed_varlen(seed, n_decode=0, **kw)
    w.name = "mixed_varlen_prefill"
    return w


def chunked_prefill_long(seed: int = SEED_BASE + 10, *, prior=32256, chunk=512,
                         num_blocks=2080) -> Workload:
    """One 512-row prefill chunk of a 32768-token prompt (prior 32256 keys):
    32 query / 8 KV heads, D=128, B=16, bf16 (an extension workload: the
    long-context chunked prefill the continuous-batching configuration's
    chunks are drawn from, at the long-context configuration's length)."""
    w = varlen_workload("chunked_prefill_long", [(prior, chunk)], num_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=num_blocks, dtype="bf16", seed=seed)
    return w


def fp8_cache(w: Workload, seed: int = SEED_BASE + 9) -> Workload:
    """The same workload with E4M3 caches: one K and one V scale per KV head,
    drawn so that the N(0,1) data spans 3.5-5 sigma of the 448 code range
    (the largest values saturate, as in a calibrated cache)."""
    rng = np.random.default_rng(seed)
    hk = w.num_kv_heads
    w.kv_dtype = "fp8"
    w.k_scale = (rng.uniform(3.5, 5.0, size=hk) / 448.0).astype(np.float32)
    w.v_scale = (rng.uniform(3.5, 5.0, size=hk) / 448.0).astype(np.float32)
    w.name = w.name + "_fp8"
    return w


def beam_search(seed: int = SEED_BASE + 6, *, width=4, prompt_len=600, steps=40,
                num_blocks=2048) -> Workload:
    """bf16 beam search (an extension workload, not among the five
    configurations): beam width 4 over a 600-token prompt for 40 decoding
    steps, 32 query / 8 KV heads, D=128, B=16."""
    return beam_search_workload("beam_search", width=width, prompt_len=prompt_len, steps=steps,
                                num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                num_blocks=num_blocks, dtype="bf16", seed=seed)


def prefix_cache(seed: int = SEED_BASE + 8, *, tenants=8, sys_len=1000, user_lo=32,
                 user_hi=512, arrivals=16, steps=8, lifetime=4, gen_lo=16,
                 gen_hi=128) -> Workload:
    """bf16 decode with prefix caching (an extension workload, not among the
    five configurations): 8 tenants with 1000-token system prompts, user
    messages of 32-512 tokens, 16 arrivals per step over 8 steps, each
    request living 4 steps and generating 16-128 tokens per step; the final
    decode step covers the 64 live requests.  32 query / 8 KV heads, D=128,
    B=16."""
    return prefix_cache_workload("prefix_cache", tenants=tenants, sys_len=sys_len,
                                 user_lo=user_lo, user_hi=user_hi, arrivals=arrivals,
                                 steps=steps, lifetime=lifetime, gen_lo=gen_lo, gen_hi=gen_hi,
                                 num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                 dtype="bf16", seed=seed)


FULL = {
    "tiny_f32_decode": tiny_f32,
    "gqa_decode_b32": gqa_decode,
    "long_ctx_decode": long_context,
    "parallel_sampling_cow": parallel_sampling,
    "mixed_varlen": mixed_varlen,
    # the prefill segments of mixed_varlen alone
    "mixed_varlen_prefill": mixed_varlen_prefill,
    "chunked_prefill_long": chunked_prefill_long,
    # parity variant of parallel_sampling_cow whose prompt ends inside a
    # block, so copy-on-write copies happen in the measured step
    "parallel_sampling_cow_1020": parallel_sampling_unaligned,
    # one GPU's share of long_ctx_decode under 8-way tensor parallelism
    "long_ctx_decode_tp8_share": long_context_tp8_share,
    # extensions, not among the five configurations: beam search, prefix
    # caching and E4M3-cache variants
    "beam_search": beam_search,
    "prefix_cache": prefix_cache,
    "gqa_decode_b32_fp8": lambda: fp8_cache(gqa_decode()),
    "long_ctx_decode_fp8": lambda: fp8_cache(long_context()),
    "mixed_varlen_fp8": lambda: fp8_cache(mixed_varlen()),
}


def reduced(name: str, seed: Optional[int] = None) -> Workload:
    """Smaller twin of a named workload, same structure, sized so the fp64 CPU
    oracle computes every output in a few seconds while still spanning
    several partitions and ragged block / partition tails."""
    s = (SEED_BASE + 100) if seed is None else seed
    if name == "tiny_f32_decode":
        return tiny_f32(s)
    if name == "gqa_decode_b32":
        return gqa_decode(s, batch=6, lo=1, hi=1300, num_blocks=1024)
    if name == "long_ctx_decode":
        return long_context(s, batch=2, ctx=3000, num_blocks=512)
    if name == "parallel_sampling_cow":
        return parallel_sampling(s, groups=3, members=4, prefix_len=100, suffix_hi=40,
                                 num_blocks=256)
    if name == "mixed_varlen":
        return mixed_varlen(s, n_prefill=2, chunk=70, prior_hi=300, n_decode=9,
                            median=120.0, lo=1, hi=700, num_blocks=512)
    if name == "chunked_prefill_long":
        return chunked_prefill_long(s, prior=1800, chunk=100, num_blocks=128)
    if name == "parallel_sampling_cow_1020":
        return parallel_sampling_unaligned(s, groups=3, members=4, prefix_len=45, suffix_hi=40,
                                           num_blocks=256)
    if name == "long_ctx_decode_tp8_share":
        return long_context_tp8_share(s, batch=2, ctx=3000, num_blocks=512)
    if name == "mixed_varlen_prefill":
        return mixed_varlen_prefill(s, chunk=70, prior_hi=300, num_blocks=512)
    if name == "beam_search":
        return beam_search(s, width=4, prompt_len=37, steps=23, num_blocks=128)
    if name == "prefix_cache":
        return prefix_cache(s, tenants=3, sys_len=45, user_lo=1, user_hi=40, arrivals=4,
                            steps=6, lifetime=2, gen_lo=1, gen_hi=20)
    if name.endswith("_fp8"):
        return fp8_cache(reduced(name[: -len("_fp8")], seed))
    raise KeyError(name)
