"""Oracle block manager: logical KV blocks mapped onto a pool of physical blocks.

Test infrastructure only (see `oracle/__init__.py`).

What the pages fix, and where:

* The KV cache is cut into fixed-size blocks of B token slots (16 by default,
  4 in the worked example); each request keeps a block table from logical
  block index to physical block number, and physical blocks need not be
  contiguous ("vLLM" documentation page, section "PagedAttention"; SourceAIX
  page, §5.1.1).
* Allocation is on demand.  A request starts with an empty table; its
  prompt's tokens fill blocks in order (allocating as each block runs out);
  at every decode token, if the current block is full a new physical block
  is allocated and appended to the table, then the token's K/V is stored in
  the current block.  When the request finishes, all its blocks are released
  and the table deleted ("vLLM" page, section "算法流程", steps 1–4).
* Each physical block carries a reference count: +1 when another request
  reuses it, −1 when a user finishes, freed at 0 ("vLLM" page, section
  "引用计数管理").
* Copy-on-write: a request about to write a token into a block whose
  reference count exceeds 1 gets a new block, the old contents are copied
  into it, the token is written there, its table is repointed, and the old
  block's count drops by 1 ("vLLM" page, section "写时复制"; SourceAIX page
  §5.2.1, where sample A1 moves to new block 3 and block 1 stays with A2).
* A slot is the unit one token occupies; a block holds several slots
  (CSDN "vLLM 0.10.0" page, §3.3).

Readings where the pages are silent (each listed in the design doc):

* slot = physical_block * B + (position mod B).
* The free pool hands out blocks from the front of a list whose initial
  order is given (a seeded permutation in the workloads); released blocks go
  to the back (the CSDN page keeps free blocks in a linked list with LRU
  eviction; first-in first-out is its plainest form).
* A block is allocated when a token needs a slot and the last block is full
  or absent (lazy; the "算法流程" decode rule), so after the 8th token of a
  7+1 token request at B=4 the table still has 2 blocks, and the 9th token
  opens the third.
* Within one operation list, operations apply in order; the first sharer to
  write into a shared block copies it, and the last remaining user writes in
  place.
* A write into a full shared block never copies: the token goes to a fresh
  block.

Prefix caching ("vLLM" page, sections "共享前缀检测" and "Prefix Caching";
CSDN page §3.3 for the LRU list):

* A request that arrives with its prompt (`new_prefix`) looks its prompt's
  prefixes up in a cache; on a hit it reuses the cached KV blocks directly
  (reference count +1) and those tokens skip prefill; on a miss it computes
  them as usual and the result is cached.
* Readings: the unit of caching is a full block (sharing is per physical
  block), so the key of logical block i is the prompt's whole token prefix
  up to the end of that block, tokens [0, (i+1)B); only the prompt's full
  blocks are cached.  The longest run of leading blocks found in the cache
  is reused.  A block enters the cache when its prompt's tokens fill it,
  unless that prefix is cached already.  A released block keeps its cache
  entry while it waits in the free list and can still be hit (then it
  leaves the list); the list is least recently released first, so the
  block allocation takes from its front is the one evicted (its entry is
  dropped).  A forked request offers no prefixes of its own (its parent's
  blocks are the ones it shares).
* Keys here are the token tuples themselves, so two prefixes match only if
  they are equal.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    """The pool has no free physical block left."""


class OracleBlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if block_size <= 0 or num_blocks < 0:
            raise ValueError("bad pool shape")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.free: deque = deque(order)
        self.ref_count: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.num_tokens: Dict[int, int] = {}
        # prefix cache: token prefix -> block, and each cached block's prefix
        self.cache: Dict[tuple, int] = {}
        self.key_of: Dict[int, tuple] = {}
        self.prompt_keys: Dict[int, List[tuple]] = {}

    # -- pool ---------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free physical block")
        b = self.free.popleft()
        assert self.ref_count[b] == 0
        if b in self.key_of:
            # the least recently released cached block: evict it
            del self.cache[self.key_of.pop(b)]
        self.ref_count[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref_count[b] -= 1
        assert self.ref_count[b] >= 0
        if self.ref_count[b] == 0:
            self.free.append(b)

    # -- requests -----------------------------------------------------------
    def new(self, sid: int) -> None:
        """A request arrives: its block table starts empty."""
        if sid in self.tables:
            raise ValueError(f"sequence {sid} exists")
        self.tables[sid] = []
        self.num_tokens[sid] = 0

    def new_prefix(self, sid: int, tokens) -> int:
        """A request arrives with its prompt's token ids.

        Reuses the longest run of leading full blocks whose prefixes are
        cached (reference count +1; a block waiting in the free list leaves
        it) and returns how many prompt tokens that covers; those tokens
        skip prefill.  The caller then appends the remaining prompt tokens.
        """
        if sid in self.tables:
            raise ValueError(f"sequence {sid} exists")
        B = self.block_size
        tokens = tuple(int(t) for t in tokens)
        keys = [tokens[: (i + 1) * B] for i in range(len(tokens) // B)]
        table = []
        for key in keys:
            if key not in self.cache:
                break
            b = self.cache[key]
            if self.ref_count[b] == 0:
                self.free.remove(b)
            self.ref_count[b] += 1
            table.append(b)
        self.tables[sid] = table
        self.num_tokens[sid] = len(table) * B
        self.prompt_keys[sid] = keys
        return len(table) * B

    def fork(self, parent: int, child: int) -> None:
        """child reuses every physical block of parent (reference count +1)."""
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        tbl = list(self.tables[parent])
        for b in tbl:
            self.ref_count[b] += 1
        self.tables[child] = tbl
        self.num_tokens[child] = self.num_tokens[parent]

    def append_one(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Give the next token of sid a slot.

        Returns (slot, copy) where copy is (src_block, dst_block) when the
        write forced a copy-on-write, else None.
        """
        B = self.block_size
        tbl = self.tables[sid]
        n = self.num_tokens[sid]
        copy = None
        if n == len(tbl) * B:
            # current block full (or no block yet): allocate, update the table
            tbl.append(self._take())
        elif self.ref_count[tbl[-1]] > 1:
            # shared block: new block, copy old contents, repoint, old count -1
            old = tbl[-1]
            new = self._take()
            tbl[-1] = new
            self.ref_count[old] -= 1
            copy = (old, new)
        blk = tbl[-1]
        self.num_tokens[sid] = n + 1
        if (n + 1) % B == 0:
            # block (n+1)/B - 1 is now full: if it holds a prompt prefix, cache it
            keys = self.prompt_keys.get(sid, [])
            i = (n + 1) // B - 1
            if i < len(keys) and keys[i] not in self.cache:
                assert blk not in self.key_of
                self.cache[keys[i]] = blk
                self.key_of[blk] = keys[i]
        return blk * B + n % B, copy

    def append(self, sid: int, n: int):
        slots, copies = [], []
        for _ in range(n):
            s, c = self.append_one(sid)
            slots.append(s)
            if c is not None:
                copies.append(c)
        return slots, copies

    def free_seq(self, sid: int) -> None:
        """Request finished: release every block (count −1) and drop the table."""
        for b in self.tables.pop(sid):
            self._release(b)
        del self.num_tokens[sid]
        self.prompt_keys.pop(sid, None)

    # -- views --------------------------------------------------------------
    def filled(self, sid: int) -> List[int]:
        """Per logical block, how many of its slots hold a token (# filled)."""
        B, n = self.block_size, self.num_tokens[sid]
        return [min(B, n - i * B) for i in range(len(self.tables[sid]))]

    def apply(self, ops, rows=None):
        """Apply a list of script operations; return (slots, copies) in order.

        Each "append" op brings n K/V rows and each ("prompt", sid, tokens)
        op len(tokens) rows, in op order; a prompt's cached tokens are not
        written.  When `rows` is a list, it receives the index of the row
        behind each returned slot.
        """
        slots, copies = [], []
        row = 0
        for op in ops:
            kind = op[0]
            if kind == "new":
                self.new(op[1])
            elif kind == "fork":
                self.fork(op[1], op[2])
            elif kind == "append":
                s, c = self.append(op[1], op[2])
                slots += s
                copies += c
                if rows is not None:
                    rows += range(row, row + op[2])
                row += op[2]
            elif kind == "prompt":
                n = len(op[2])
                hit = self.new_prefix(op[1], op[2])
                s, c = self.append(op[1], n - hit)
                slots += s
                copies += c
                if rows is not None:
                    rows += range(row + hit, row + n)
                row += n
            elif kind == "free":
                self.free_seq(op[1])
            else:
                raise ValueError(f"unknown op {op!r}")
        return slots, copies
