"""Pins for the oracle's prefix cache (OracleBlockManager.new_prefix).

The rules come from the "vLLM" documentation page (sections 共享前缀检测 and
Prefix Caching: hash a prompt's prefix, reuse the cached KV on a hit with
reference count +1 and skip that prefill, compute and cache on a miss) and
the CSDN "vLLM 0.10.0 flow" page §3.3 (free blocks in a doubly linked list,
oldest evicted first).

Pins:
* a worked example at B = 4 whose block numbers, cached-token counts,
  reference counts and evictions were derived by hand from those rules;
* a prefix key must be the whole prefix, not one block's tokens (two prompts
  whose blocks hold the same tokens in another order share nothing);
* a content check on random scripts: a token store written through the
  returned slots must read back, through every live request's table, the
  exact token ids of that request (prompt, then generated), so a wrong hit,
  a stale key after eviction or a write into a shared block fails;
* planted mistakes (block-local keys, no eviction) are caught.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import run
from oracle.block_manager import OracleBlockManager, OutOfBlocks
from tests.libutil import without_prefix_cache


def _prompt(bm, sid, tokens):
    hit = bm.new_prefix(sid, tokens)
    slots, copies = bm.append(sid, len(tokens) - hit)
    assert not copies
    return hit, slots


def test_worked_example_hits_reuse_and_lru_eviction(cls=OracleBlockManager):
    bm = cls(8, 4)                                  # free list 0..7
    r1 = list(range(1, 11))                         # 10 tokens: blocks 0, 1 full, 2 partial
    assert _prompt(bm, 1, r1) == (0, list(range(0, 10)))
    assert bm.tables[1] == [0, 1, 2]
    # request 2 shares the first 8 tokens: two blocks reused, 3 tokens computed
    hit, slots = _prompt(bm, 2, list(range(1, 9)) + [99, 98, 97])
    assert (hit, slots) == (8, [12, 13, 14])
    assert bm.tables[2] == [0, 1, 3] and bm.ref_count[:4] == [2, 2, 1, 1]
    # request 3 shares only the first block; its own second block gets cached
    hit, slots = _prompt(bm, 3, [1, 2, 3, 4, 50, 51, 52, 53])
    assert (hit, slots) == (4, [16, 17, 18, 19]) and bm.tables[3] == [0, 4]
    assert bm.ref_count[0] == 3 and list(bm.free) == [5, 6, 7]
    # releasing keeps the cached blocks (1 and 3 and 2 go to the back)
    bm.free_seq(1)
    bm.free_seq(2)
    assert list(bm.free) == [5, 6, 7, 2, 1, 3]
    # a prompt entirely in the cache: nothing to prefill; block 1 leaves the free list
    assert _prompt(bm, 4, list(range(1, 9))) == (8, [])
    assert bm.tables[4] == [0, 1] and list(bm.free) == [5, 6, 7, 2, 3]
    assert bm.append(4, 1) == ([20], [])            # the decode token opens block 5
    bm.free_seq(3)
    bm.free_seq(4)
    assert list(bm.free) == [6, 7, 2, 3, 4, 0, 1, 5]
    # a 20-token miss takes 6, 7, 2, 3, 4: block 4 is evicted on the way
    hit, slots = _prompt(bm, 5, list(range(100, 120)))
    assert hit == 0 and bm.tables[5] == [6, 7, 2, 3, 4]
    assert list(bm.free) == [0, 1, 5]
    # block 0 is still cached, block 4's prefix is gone; allocation then
    # takes block 1 from the front and evicts the 8-token prefix
    hit, slots = _prompt(bm, 6, [1, 2, 3, 4, 50, 51, 52, 53])
    assert hit == 4 and bm.tables[6] == [0, 1] and list(bm.free) == [5]
    assert _prompt(bm, 7, list(range(1, 9)))[0] == 4
    # request 5's five full blocks are cached: a later copy of its prompt hits all
    bm.free_seq(7)
    bm.free_seq(6)
    bm.free_seq(5)
    assert _prompt(bm, 8, list(range(100, 120)) + [7])[0] == 20


def test_key_is_the_whole_prefix(cls=OracleBlockManager):
    bm = cls(8, 4)
    _prompt(bm, 0, [1, 1, 1, 1, 2, 2, 2, 2])
    # same blocks' tokens, other order: the first block (2,2,2,2) is not a cached prefix
    assert _prompt(bm, 1, [2, 2, 2, 2, 1, 1, 1, 1])[0] == 0
    # a prefix shorter than a block is never shared
    assert _prompt(bm, 2, [1, 1, 1])[0] == 0
    assert bm.tables[2] != [bm.tables[0][0]]


def test_duplicate_prompts_in_flight_cache_once():
    bm = OracleBlockManager(8, 4)
    bm.new_prefix(0, [5] * 8)
    bm.new_prefix(1, [5] * 8)           # nothing cached yet: both miss
    bm.append(0, 8)
    bm.append(1, 8)                     # same prefix already cached by request 0
    assert sorted(bm.cache.values()) == sorted(bm.tables[0])
    assert _prompt(bm, 2, [5] * 8 + [6]) == (8, [4 * bm.tables[2][2]])
    assert bm.tables[2][:2] == bm.tables[0]


def test_fork_shares_but_does_not_offer():
    bm = OracleBlockManager(8, 4)
    bm.new_prefix(0, [3] * 6)
    bm.append(0, 4)
    bm.fork(0, 1)                       # child shares the cached block
    bm.append(1, 4)                     # child's tokens 4..7 fill its second block
    assert len(bm.cache) == 1
    assert _prompt(bm, 2, [3] * 8)[0] == 4


class _Store:
    """Token ids written through slots, read back through block tables."""

    def __init__(self, bm):
        self.bm = bm
        self.slot = {}
        self.truth = {}

    def prompt(self, sid, tokens):
        hit = self.bm.new_prefix(sid, tokens)
        self.truth[sid] = list(tokens[:hit])
        self.append(sid, tokens[hit:])
        return hit

    def append(self, sid, ids):
        # token by token, so a pool that runs dry part-way leaves the store in step
        B = self.bm.block_size
        for t in ids:
            slot, copy = self.bm.append_one(sid)
            if copy is not None:
                src, dst = copy
                for j in range(B):
                    if src * B + j in self.slot:
                        self.slot[dst * B + j] = self.slot[src * B + j]
            self.slot[slot] = t
            self.truth[sid].append(t)

    def fork(self, a, b):
        self.bm.fork(a, b)
        self.truth[b] = list(self.truth[a])

    def free(self, sid):
        self.bm.free_seq(sid)
        del self.truth[sid]

    def check(self):
        B = self.bm.block_size
        for sid, toks in self.truth.items():
            tbl = self.bm.tables[sid]
            got = [self.slot.get(tbl[p // B] * B + p % B) for p in range(len(toks))]
            assert got == toks, sid


_TEMPLATES = [[7] * 9, [1, 2, 3, 4, 5, 6, 7, 8], [7] * 4 + [1] * 4, [2] * 12]


def _run_random(bm_cls, ops, B, nb=24):
    bm = bm_cls(nb, B, list(reversed(range(nb))))
    store = _Store(bm)
    fresh = 1000
    for kind, a, b, n in ops:
        live = set(store.truth)
        try:
            if kind == "prompt" and a not in live:
                toks = _TEMPLATES[b % len(_TEMPLATES)][: 4 + 2 * n] + [fresh + j for j in range(n % 3)]
                fresh += 3
                store.prompt(a, toks)
            elif kind == "fork" and a in live and b not in live:
                store.fork(a, b)
            elif kind == "append" and a in live:
                store.append(a, [fresh + j for j in range(n)])
                fresh += n
            elif kind == "free" and a in live:
                store.free(a)
        except OutOfBlocks:
            # the oracle fails part-way: drop the request whose append failed
            store.free(a)
        store.check()
        for key, blk in bm.cache.items():
            assert bm.key_of[blk] == key and len(key) % B == 0
        assert len(bm.free) + sum(1 for r in bm.ref_count if r) == nb
    return bm


_OPS = st.lists(st.tuples(st.sampled_from(["prompt", "prompt", "fork", "append", "free"]),
                          st.integers(0, 5), st.integers(0, 5), st.integers(0, 6)),
                max_size=60)


@settings(max_examples=150, deadline=None)
@given(_OPS, st.sampled_from([2, 4]))
def test_random_scripts_read_back_their_own_tokens(ops, B):
    _run_random(OracleBlockManager, ops, B)


class _LocalKeys(OracleBlockManager):
    """Planted mistake: a block's key is its own tokens, not the whole prefix."""

    def new_prefix(self, sid, tokens):
        B = self.block_size
        tokens = tuple(int(t) for t in tokens)
        n = super().new_prefix(sid, [])
        self.prompt_keys[sid] = [tokens[i * B:(i + 1) * B] for i in range(len(tokens) // B)]
        for key in self.prompt_keys[sid]:
            if key not in self.cache:
                break
            b = self.cache[key]
            if self.ref_count[b] == 0:
                self.free.remove(b)
            self.ref_count[b] += 1
            self.tables[sid].append(b)
        self.num_tokens[sid] = len(self.tables[sid]) * B
        return self.num_tokens[sid] + n


class _NoEviction(OracleBlockManager):
    """Planted mistake: allocation reuses a cached block but keeps its key."""

    def _take(self):
        if not self.free:
            raise OutOfBlocks("no free physical block")
        b = self.free.popleft()
        self.ref_count[b] = 1
        return b


@pytest.mark.parametrize("cls", [_LocalKeys, _NoEviction])
def test_planted_mistakes_are_caught(cls):
    with pytest.raises(AssertionError):
        test_key_is_the_whole_prefix(cls)
        test_worked_example_hits_reuse_and_lru_eviction(cls)


class _Counting(OracleBlockManager):
    evictions = 0

    def _take(self):
        if self.free and self.free[0] in self.key_of:
            _Counting.evictions += 1
        return super()._take()


def test_multi_tenant_workload_hits_evicts_and_attends_the_same():
    w = synth.reduced("prefix_cache")
    _Counting.evictions = 0
    orig = run.OracleBlockManager
    run.OracleBlockManager = _Counting
    try:
        st = run.run_script(w)
    finally:
        run.OracleBlockManager = orig
    assert st.prefill_skipped > 0 and _Counting.evictions > 0
    assert st.prefill_skipped % w.block_size == 0
    # skipping the cached prefill changes nothing the step attends to
    st2 = run.run_script(without_prefix_cache(w))
    assert st2.prefill_skipped == 0
    assert np.array_equal(run.attend(w, st), run.attend(w, st2))
    # and the prefix cache used fewer blocks than computing every prompt
    used = lambda s: sum(1 for r in s.bm.ref_count if r)
    assert used(st) < used(st2)
