"""Drive a serving script through libpa: the host block manager decides slots,
block tables and copy-on-write pairs; the HIP kernels copy blocks, write K/V
and attend.

A script is a list of steps; each step holds operations ("new", sid),
("fork", parent, child), ("append", sid, n), ("prompt", sid, tokens),
("free", sid) and the K/V rows of its appended and prompt tokens in order.
A prompt starts its sequence through the prefix cache; the rows of its
cached tokens are not written (their K/V is already in the pool).  `ScriptRunner` applies the history steps
(filling the cache, untimed) and prepares the final step, whose
`run_step()` is the measured hot path: copy-on-write block copies, the
slot_mapping scatter of the step's tokens, then decode (one query row per
sequence) or varlen attention (query rows delimited by query_start_loc).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from . import (LAYOUT_PLAIN, BlockManager, cache_dims, cache_write, copy_blocks, decode,
               decode_workspace_bytes, varlen, varlen_workspace_bytes)


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, dtype_name: str, device):
    """Host storage array (uint16 bf16 bits or float32) -> device tensor."""
    torch = _torch()
    if dtype_name == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host_bits(t) -> np.ndarray:
    """Device tensor -> host storage array (uint16 bits for bf16, uint8 codes
    for float8_e4m3fn, float32)."""
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.float().cpu().numpy()


@dataclasses.dataclass
class FinalStep:
    k: object
    v: object
    slot_mapping: object
    copy_pairs: Optional[object]   # [n][2] int32 or None
    q: object
    block_tables: object
    context_lens: object
    query_start_loc: object
    out: object
    workspace: Optional[object]
    max_context_len: int
    max_query_len: int
    host_slots: np.ndarray
    host_copies: List[Tuple[int, int]]
    host_tables: np.ndarray
    host_lens: np.ndarray
    host_qsl: np.ndarray
    # launch row i is batch row order[i] (None: batch order); the device
    # tensors above (q, k, v, slot_mapping, block_tables, context_lens, out)
    # are in launch order, the host_* arrays in batch order
    order: Optional[np.ndarray] = None


class ScriptRunner:
    def __init__(self, w, device="cuda", fill: Optional[str] = "canary",
                 table_width: Optional[int] = None, layout: int = LAYOUT_PLAIN,
                 group_prefixes: bool = False):
        torch = _torch()
        self.w = w
        # order a decode step's rows by their first block, so that requests
        # sharing a prompt prefix sit next to each other and the decode
        # kernels read the prefix once for all of them (a scheduler's choice
        # of batch order; outputs are the same up to rounding)
        self.group_prefixes = group_prefixes
        self.device = torch.device(device)
        self.tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        # FP8 caches (w.kv_dtype == "fp8"): E4M3 codes with per-KV-head scales;
        # q and the new tokens' k, v stay in w.dtype (bf16)
        self.fp8 = getattr(w, "kv_dtype", None) == "fp8"
        cdtype = torch.float8_e4m3fn if self.fp8 else self.tdtype
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        self.k_cache = torch.empty(shape, dtype=cdtype, device=self.device)
        self.v_cache = torch.empty(shape, dtype=cdtype, device=self.device)
        self.kv_scales = None
        if self.fp8:
            self.kv_scales = (torch.from_numpy(np.asarray(w.k_scale, np.float32)).to(self.device),
                              torch.from_numpy(np.asarray(w.v_scale, np.float32)).to(self.device))
        if fill == "canary":
            # NaN in every slot no token owns
            if self.fp8:
                self.k_cache.view(torch.uint8).fill_(0x7F)
                self.v_cache.view(torch.uint8).fill_(0x7F)
            elif w.dtype == "bf16":
                self.k_cache.view(torch.int16).fill_(0x7FC1)
                self.v_cache.view(torch.int16).fill_(0x7FC1)
            else:
                self.k_cache.view(torch.int32).fill_(0x7FC00001)
                self.v_cache.view(torch.int32).fill_(0x7FC00001)
        elif fill == "zero":
            self.k_cache.zero_()
            self.v_cache.zero_()
        self.bm = BlockManager(w.num_blocks, w.block_size, w.free_order)
        self.prefill_skipped = 0   # prompt tokens served by the prefix cache
        self.table_width = table_width
        self.layout = layout   # KV head order inside a slot (pa_layout)
        self.dims = cache_dims(self.k_cache, w.num_heads, self.kv_scales, layout)

    # -- host side -----------------------------------------------------------
    def host_step(self, step) -> Tuple[np.ndarray, List[Tuple[int, int]], Optional[np.ndarray]]:
        """Block-manager work of a step: (slots, copy pairs, rows), where rows
        lists the step's K/V rows behind the slots, or is None when every row
        is written in order."""
        n = sum(op[2] if op[0] == "append" else len(op[2]) if op[0] == "prompt" else 0
                for op in step.ops)
        slots = np.empty(n, dtype=np.int32)
        rows = np.empty(n, dtype=np.int64)
        copies = []
        i = r = 0
        for op in step.ops:
            kind = op[0]
            if kind == "new":
                self.bm.new(op[1])
            elif kind == "fork":
                self.bm.fork(op[1], op[2])
            elif kind == "free":
                self.bm.free(op[1])
            elif kind in ("append", "prompt"):
                if kind == "prompt":
                    hit = self.bm.new_prefix(op[1], op[2])
                    self.prefill_skipped += hit
                    r += hit
                    cnt = len(op[2]) - hit
                else:
                    cnt = op[2]
                cp = self.bm.append_into(op[1], cnt, slots[i:i + cnt])
                if cp is not None:
                    copies.append(cp)
                rows[i:i + cnt] = np.arange(r, r + cnt)
                i += cnt
                r += cnt
            else:
                raise ValueError(f"unknown op {op!r}")
        if i == n:
            return slots, copies, None
        return slots[:i], copies, rows[:i]

    def _pairs(self, copies):
        torch = _torch()
        if not copies:
            return None
        return torch.tensor(copies, dtype=torch.int32, device=self.device).reshape(-1, 2)

    def apply(self, step) -> None:
        """Host bookkeeping, then copies and writes on the device (current stream)."""
        torch = _torch()
        slots, copies, rows = self.host_step(step)
        pairs = self._pairs(copies)
        if pairs is not None:
            copy_blocks(self.k_cache, self.v_cache, pairs)
        if len(slots):
            sk, sv = (step.k, step.v) if rows is None else (step.k[rows], step.v[rows])
            k = to_device(sk, self.w.dtype, self.device)
            v = to_device(sv, self.w.dtype, self.device)
            sm = torch.from_numpy(slots).to(self.device)
            cache_write(k, v, sm, self.k_cache, self.v_cache, kv_scales=self.kv_scales,
                        layout=self.layout)

    def run_history(self) -> None:
        for step in self.w.history:
            self.apply(step)

    # -- the measured step ----------------------------------------------------
    def prepare_final(self, partition_size: Optional[int] = None) -> FinalStep:
        torch = _torch()
        w = self.w
        if any(op[0] == "prompt" for op in w.final.ops):
            raise ValueError("the measured step appends tokens; prompts arrive before it")
        slots, copies, _ = self.host_step(w.final)
        batch = [int(s) for s in w.batch]
        B = w.block_size
        width = self.table_width
        if width is None:
            width = max([-(-self.bm.num_tokens(s) // B) for s in batch] + [1])
        tables, lens = self.bm.batch_tables(batch, width)
        qlen = {s: 0 for s in batch}
        for op in w.final.ops:
            if op[0] == "append":
                qlen[op[1]] += op[2]
        qsl = np.zeros(len(batch) + 1, dtype=np.int32)
        qsl[1:] = np.cumsum([qlen[s] for s in batch])
        dev = self.device
        order = self._launch_order(batch, tables, lens)
        if order is None:
            q_h, k_h, v_h, slots_h, tables_h, lens_h = w.q, w.final.k, w.final.v, slots, tables, lens
        else:  # the step's rows (one appended token each) follow the batch
            q_h, k_h, v_h = w.q[order], w.final.k[order], w.final.v[order]
            slots_h, tables_h, lens_h = slots[order], tables[order], lens[order]
        q = to_device(q_h, w.dtype, dev)
        max_ctx = int(lens.max()) if len(lens) else 0
        ps = w.partition_size if partition_size is None else partition_size
        ws = None
        if w.kind == "decode":
            need = decode_workspace_bytes(self.dims, len(batch), max_ctx, ps)
        else:
            need = varlen_workspace_bytes(self.dims, len(batch), int(qsl[-1]),
                                          int(max(qlen.values())) if qlen else 0, max_ctx)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        fin = FinalStep(
            k=to_device(k_h, w.dtype, dev), v=to_device(v_h, w.dtype, dev),
            slot_mapping=torch.from_numpy(np.ascontiguousarray(slots_h)).to(dev),
            copy_pairs=self._pairs(copies),
            q=q, block_tables=torch.from_numpy(np.ascontiguousarray(tables_h)).to(dev),
            context_lens=torch.from_numpy(np.ascontiguousarray(lens_h)).to(dev),
            query_start_loc=torch.from_numpy(qsl).to(dev), out=torch.empty_like(q),
            workspace=ws, max_context_len=max_ctx,
            max_query_len=int(max(qlen.values())) if qlen else 0,
            host_slots=slots, host_copies=copies, host_tables=tables, host_lens=lens,
            host_qsl=qsl, order=order)
        self.partition_size = ps
        return fin

    def _launch_order(self, batch, tables, lens) -> Optional[np.ndarray]:
        """Rows stably sorted by first block (empty rows first), when
        group_prefixes is set and the step is a decode step whose rows each
        append one token in batch order; None when that is the batch order."""
        w = self.w
        if not self.group_prefixes or w.kind != "decode" or len(batch) < 2:
            return None
        appends = [(op[1], op[2]) for op in w.final.ops if op[0] == "append"]
        if [int(s) for s, _ in appends] != batch or any(n != 1 for _, n in appends):
            return None
        if any(op[0] not in ("append",) for op in w.final.ops):
            return None
        key = np.where(lens > 0, tables[:, 0], -1).astype(np.int64)
        order = np.argsort(key, kind="stable")
        return None if (order == np.arange(len(order))).all() else order

    def out_in_batch_order(self, fin: FinalStep):
        """The step's output rows in batch order (a device gather when the
        launch order differs)."""
        if fin.order is None:
            return fin.out
        torch = _torch()
        inv = np.empty_like(fin.order)
        inv[fin.order] = np.arange(len(fin.order))
        return fin.out.index_select(0, torch.from_numpy(inv).to(fin.out.device))

    def run_step(self, fin: FinalStep, k_cache=None, v_cache=None) -> None:
        """The hot path of one step: CoW copies, K/V scatter, attention."""
        kc = self.k_cache if k_cache is None else k_cache
        vc = self.v_cache if v_cache is None else v_cache
        if fin.copy_pairs is not None:
            copy_blocks(kc, vc, fin.copy_pairs)
        if fin.slot_mapping.numel():
            cache_write(fin.k, fin.v, fin.slot_mapping, kc, vc, kv_scales=self.kv_scales,
                        layout=self.layout)
        self.attend(fin, kc, vc)

    def attend(self, fin: FinalStep, k_cache=None, v_cache=None) -> None:
        kc = self.k_cache if k_cache is None else k_cache
        vc = self.v_cache if v_cache is None else v_cache
        w = self.w
        if w.kind == "decode":
            decode(fin.q, kc, vc, fin.block_tables, fin.context_lens, w.scale, fin.out,
                   fin.max_context_len, self.partition_size, fin.workspace,
                   kv_scales=self.kv_scales, layout=self.layout)
        else:
            varlen(fin.q, fin.query_start_loc, fin.context_lens, kc, vc, fin.block_tables,
                   w.scale, fin.out, fin.max_query_len, fin.max_context_len, fin.workspace,
                   kv_scales=self.kv_scales, layout=self.layout)
