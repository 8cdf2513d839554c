"""Pins for the oracle block manager: the pages' worked examples and invariants."""
import json
import math
import os

import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import OracleBlockManager, OutOfBlocks

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _order(head, n):
    return list(head) + [b for b in range(n) if b not in head]


def test_single_request_worked_example():
    g = _gold("sourceaix_single_request.json")
    B = g["block_size"]
    bm = OracleBlockManager(16, B, _order(g["free_order_head"], 16))
    bm.new(0)
    slots, copies = bm.append(0, g["prompt_tokens"])
    assert bm.tables[0] == g["after_prefill"]["table"]
    assert bm.filled(0) == g["after_prefill"]["filled"]
    assert copies == []
    # prompt slots run through block 7 then block 1 (one reservation slot left)
    assert slots == [7 * B + i for i in range(4)] + [1 * B + i for i in range(3)]
    s, c = bm.append_one(0)
    assert c is None and s == 1 * B + 3
    assert bm.tables[0] == g["after_decode_1"]["table"]
    assert bm.filled(0) == g["after_decode_1"]["filled"]
    bm.append_one(0)
    assert len(bm.tables[0]) == g["after_decode_2"]["num_logical_blocks"]
    assert bm.filled(0) == g["after_decode_2"]["filled"]


def test_parallel_sampling_copy_on_write_example():
    g = _gold("sourceaix_parallel_sampling.json")
    B = g["block_size"]
    bm = OracleBlockManager(16, B, _order(g["free_order_head"], 16))
    a1, a2 = 1, 2
    bm.new(a1)
    bm.append(a1, g["prompt_tokens"])
    bm.fork(a1, a2)
    exp = g["after_fork"]
    assert bm.tables[a1] == exp["A1"] and bm.tables[a2] == exp["A2"]
    for b, r in exp["ref_count"].items():
        assert bm.ref_count[int(b)] == r
    s, c = bm.append_one(a1)
    exp = g["after_A1_token"]
    assert c == tuple(exp["copy"])
    assert bm.tables[a1] == exp["A1"] and bm.tables[a2] == exp["A2"]
    for b, r in exp["ref_count"].items():
        assert bm.ref_count[int(b)] == r
    assert s == 3 * B + 3
    s, c = bm.append_one(a2)
    exp = g["after_A2_token"]
    assert c is None and s == 1 * B + 3
    assert bm.tables[a1] == exp["A1"] and bm.tables[a2] == exp["A2"]
    for b, r in exp["ref_count"].items():
        assert bm.ref_count[int(b)] == r


def test_docs_block_table_and_utilisation():
    g = _gold("vllm_docs_block_table.json")
    e = g["block_table_example"]
    bm = OracleBlockManager(64, e["block_size"], _order(e["free_order_head"], 64))
    bm.new(0)
    bm.append(0, e["tokens"])
    assert bm.tables[0] == e["table"]
    u = g["utilisation_example"]
    bm = OracleBlockManager(64, u["block_size"])
    bm.new(0)
    bm.append(0, u["tokens"])
    assert len(bm.tables[0]) == u["blocks"] == math.ceil(u["tokens"] / u["block_size"])
    assert len(bm.tables[0]) * u["block_size"] * u["bytes_per_token"] == u["allocated_bytes"]
    assert bm.filled(0) == [16] * 16  # no reserved-but-unused slot at all


def test_finish_releases_blocks_and_table():
    bm = OracleBlockManager(8, 4)
    bm.new(0)
    bm.append(0, 10)
    assert len(bm.free) == 5
    bm.free_seq(0)
    assert 0 not in bm.tables
    assert len(bm.free) == 8 and all(r == 0 for r in bm.ref_count)
    # released blocks go to the back of the pool, in table order
    assert list(bm.free) == [3, 4, 5, 6, 7, 0, 1, 2]


def test_beam_search_elimination_frees_what_only_dead_beams_held():
    # SourceAIX page §5.2.2: when the next beams come only from candidates 1
    # and 2, the eliminated candidates' blocks are freed, and so is a block
    # that only an eliminated candidate still reached (its block 4 after
    # block 8).  B = 4: prompt block P shared by all beams; beam 4 was forked
    # from beam 3 after their common block X filled; every beam then got a
    # private block.
    bm = OracleBlockManager(16, 4)
    bm.new(1)
    bm.append(1, 4)                      # P
    for b in (2, 3):
        bm.fork(1, b)
    bm.append(3, 4)                      # X (beam 3 only so far)
    bm.fork(3, 4)                        # beam 4 shares P and X
    for b in (1, 2, 3, 4):
        bm.append(b, 4)                  # one private block each
    P, X = bm.tables[1][0], bm.tables[3][1]
    priv = {b: bm.tables[b][-1] for b in (1, 2, 3, 4)}
    assert bm.ref_count[P] == 4 and bm.ref_count[X] == 2
    free_before = set(bm.free)
    # next step: two continuations of beam 1, two of beam 2; 3 and 4 die
    bm.fork(1, 5)
    bm.fork(2, 6)
    bm.free_seq(3)
    bm.free_seq(4)
    freed = set(bm.free) - free_before
    assert freed == {X, priv[3], priv[4]}
    assert bm.ref_count[P] == 4 and bm.ref_count[priv[1]] == 2 and bm.ref_count[priv[2]] == 2
    assert bm.ref_count[X] == 0
    # the new beams' tokens go to fresh blocks (the shared last blocks are full)
    for b in (1, 5, 2, 6):
        _, c = bm.append_one(b)
        assert c is None
    assert len({bm.tables[b][-1] for b in (1, 5, 2, 6)}) == 4


def test_full_shared_block_is_not_copied():
    bm = OracleBlockManager(8, 4)
    bm.new(0)
    bm.append(0, 8)
    bm.fork(0, 1)
    s, c = bm.append_one(1)
    assert c is None and bm.tables[1][:2] == bm.tables[0] and len(bm.tables[1]) == 3


def test_pool_exhaustion_raises():
    bm = OracleBlockManager(2, 4)
    bm.new(0)
    bm.append(0, 8)
    with pytest.raises(OutOfBlocks):
        bm.append_one(0)


def _check_invariants(bm):
    refs = [0] * bm.num_blocks
    for sid, tbl in bm.tables.items():
        for b in tbl:
            refs[b] += 1
        # lazy allocation: exactly ceil(n/B) blocks, so at most B-1 idle slots
        assert len(tbl) == -(-bm.num_tokens[sid] // bm.block_size)
    assert refs == bm.ref_count
    free = set(bm.free)
    assert len(free) == len(bm.free)
    for b in range(bm.num_blocks):
        assert (b in free) == (refs[b] == 0)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.sampled_from(["new", "fork", "append", "free"]),
                          st.integers(0, 5), st.integers(0, 5), st.integers(1, 9)),
                max_size=60),
       st.sampled_from([1, 2, 4, 16]))
def test_random_scripts_keep_invariants(ops, B):
    bm = OracleBlockManager(48, B, list(reversed(range(48))))
    for kind, a, b, n in ops:
        try:
            if kind == "new" and a not in bm.tables:
                bm.new(a)
            elif kind == "fork" and a in bm.tables and b not in bm.tables:
                bm.fork(a, b)
            elif kind == "append" and a in bm.tables:
                for _ in range(n):
                    slot, copy = bm.append_one(a)
                    blk = slot // B
                    # a write never lands in a block another request still uses
                    assert bm.ref_count[blk] == 1
                    assert bm.tables[a][-1] == blk
                    assert slot % B == (bm.num_tokens[a] - 1) % B
                    if copy is not None:
                        assert copy[1] == blk and bm.ref_count[copy[0]] >= 1
            elif kind == "free" and a in bm.tables:
                bm.free_seq(a)
        except OutOfBlocks:
            pass
        _check_invariants(bm)
    for sid in list(bm.tables):
        bm.free_seq(sid)
    assert len(bm.free) == bm.num_blocks and not any(bm.ref_count)
