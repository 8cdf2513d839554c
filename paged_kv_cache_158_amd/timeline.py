"""Per-wave timelines of the decode and varlen kernels (timeline build).

    python paged_kv_cache_158_amd/build.py --timeline
    python paged_kv_cache_158_amd/timeline.py decode gqa_decode_b32 [more workloads]
    python paged_kv_cache_158_amd/timeline.py varlen mixed_varlen [more workloads]

Loads `libpa_timeline.so` (the product kernels, compiled with PA_TIMELINE so
that they also write s_memrealtime stamps, a 100 MHz device clock) instead
of `libpa.so`, prepares a workload's final step as `bench.py` does (seeded
synthetic inputs, rows grouped by first block, the rotated cache layout,
pool copies rotated so that the 256 MB cache does not serve the reads),
records three launches after a warm-up and prints a summary of the last two.
Times are microseconds from the first wave's start.  The stamps cost a few
instructions per wave: the kernel times here run slightly longer than the
product's.

decode (the partition kernel of one step, balanced split): per wave, its
plan (every wave plans the whole line; the four phase stamps are, for the
plain split, lengths in registers / line length / own range / segment list
and, with shared prefixes, lengths and first entries / probes / groups /
own range), the staging of its block-table entries, and the streaming of
its chunks; per XCD, when its waves end; per SIMD and per CU, how many
waves shared one, and the streaming time of the waves that mostly had it to
themselves against the others.

varlen (one `pa_varlen` launch): per prefill workgroup, its key tiles and
microseconds per tile; when the decode workgroups start; how many
workgroups of each kind run over time.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
torch = pa = synth = ScriptRunner = None  # loaded by _load() (the timeline build)


def _load():
    """Imports torch and the package with libpa_timeline.so in place of libpa.so."""
    global torch, pa, synth, ScriptRunner
    os.environ["PA_LIBRARY"] = "libpa_timeline.so"
    sys.path.insert(0, os.path.dirname(_HERE))
    import torch as torch_
    import paged_kv_cache_158_amd as pa_
    import synth as synth_
    from paged_kv_cache_158_amd.engine import ScriptRunner as runner
    torch, pa, synth, ScriptRunner = torch_, pa_, synth_, runner

TRACE_STAMPS = 1 << 21    # buffer the library expects (decode part, then varlen part)
VARLEN_OFFSET = 1 << 20   # first stamp of the varlen records
POOLS = 6                 # rotated pool copies


def _prepare(name):
    w = synth.FULL[name]()
    r = ScriptRunner(w, torch.device("cuda:0"), fill="zero", layout=pa.LAYOUT_ROTATED,
                     group_prefixes=w.kind != "varlen")
    r.run_history()
    fin = r.prepare_final(None)
    pools = [(r.k_cache, r.v_cache)] + [(r.k_cache.clone(), r.v_cache.clone())
                                        for _ in range(POOLS - 1)]
    return w, r, fin, pools


def _record(call, trace):
    for i in range(30):
        call(i)
    torch.cuda.synchronize()
    out = []
    for rep in range(3):
        trace.zero_()
        torch.cuda.synchronize()
        pa._lib.pa_trace_set(ctypes.c_void_p(trace.data_ptr()))
        call(rep)
        pa._lib.pa_trace_set(None)
        for i in range(3):
            call(rep + 1 + i)
        torch.cuda.synchronize()
        out.append(trace.cpu().numpy().copy())
    return out[1:]


def _pct(x, q):
    return float(np.percentile(x, q))


def decode(name, trace):
    w, r, fin, pools = _prepare(name)
    shared = _has_shared_first_block(fin)
    calls = [pa.prepare_decode_append(fin.q, fin.k, fin.v, fin.slot_mapping, kc, vc,
                                      fin.block_tables, fin.context_lens, w.scale, fin.out,
                                      fin.max_context_len, 0, fin.workspace,
                                      kv_scales=r.kv_scales, partials_only=True,
                                      layout=pa.LAYOUT_ROTATED) for kc, vc in pools]
    for raw in _record(lambda i: calls[i % POOLS](), trace):
        d = raw[:VARLEN_OFFSET - VARLEN_OFFSET % 10].reshape(-1, 10)
        head = np.arange(len(d)) % w.num_kv_heads  # record y * num_kv_heads + g
        head, d = head[d[:, 0] > 0], d[d[:, 0] > 0]
        t0 = d[:, 0].min()
        us = lambda c: (d[:, c] - t0) / 100.0  # noqa: E731
        start, plan, stage, end = us(0), us(1), us(2), us(3)
        body = end - stage
        xcc = d[:, 4] & 0xF
        K = (d[:, 5] >> 32).astype(np.int64)
        print(f"== {name}: {len(d)} waves, span {end.max():.2f} us; start max {start.max():.2f}; "
              f"plan med {np.median(plan - start):.2f} max {(plan - start).max():.2f}; "
              f"staging med {np.median(stage - plan):.2f}; chunks med {np.median(K):.0f} max {K.max()}; "
              f"streaming med {np.median(body):.2f} p90 {_pct(body, 90):.2f} max {body.max():.2f}; "
              f"end med {np.median(end):.2f}")
        ph = d[:, 6:10]
        if (ph > 0).all(axis=1).any():
            m = (ph > 0).all(axis=1)
            p = [(ph[m, i] - d[m, 0]) / 100.0 for i in range(4)]
            names = (("lengths+first entries", "probes", "groups", "own range") if shared
                     else ("lengths", "line length", "own range", "segment list"))
            steps = [np.median(p[0])] + [np.median(p[i] - p[i - 1]) for i in range(1, 4)]
            steps.append(np.median((d[m, 1] - ph[m, 3]) / 100.0))
            print("   plan phases (median us): " + ", ".join(
                f"{n} {v:.2f}" for n, v in zip(names + ("to plan end",), steps)))
        for x in range(8):
            s = xcc == x
            if s.any():
                print(f"   XCD {x}: {s.sum():4d} waves, streaming med {np.median(body[s]):.2f}, "
                      f"end med {np.median(end[s]):.2f} max {end[s].max():.2f}")
        print("   streaming med per KV head: " + ", ".join(
            f"{h}: {np.median(body[head == h]):.2f}" for h in range(w.num_kv_heads) if (head == h).any()))
        print(f"   us per chunk: med {np.median(body[K > 0] / K[K > 0]):.3f}")
        # which waves had a SIMD (and a CU) to themselves while they streamed
        hw = (d[:, 4] >> 32).astype(np.int64)
        cu = _cu_ids(d[:, 4] & 0xF, hw)
        simd = cu * 4 + ((hw >> 4) & 3)
        for what, key in (("SIMD", simd), ("CU", cu)):
            per = np.unique(key, return_counts=True)[1]
            hist = ", ".join(f"{c} waves: {n}" for c, n in zip(*np.unique(per, return_counts=True)))
            peers = _peers(key, stage, end, start, end)
            one, more = peers < 0.5, peers >= 0.5
            line = f"   per {what}: {len(per)} used ({hist})"
            if one.any() and more.any():
                line += (f"; streaming med {np.median(body[one]):.2f} for the {one.sum()} waves "
                         f"with under half a peer on average, {np.median(body[more]):.2f} for the rest")
            print(line)


def _cu_ids(xcc, hw):
    """A CU's number from XCC_ID and HW_ID (CU, SH and SE fields)."""
    xcc = np.asarray(xcc).astype(np.int64)
    return (xcc << 12) | (((hw >> 13) & 7) << 8) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 15)


def _peers(key, st, en, ost, oen):
    """Per wave: the average number of other waves with the same key during
    its interval [st, en) (the others counted over [ost, oen))."""
    out = np.zeros(len(key))
    for k in np.unique(key):
        idx = np.nonzero(key == k)[0]
        for i in idx:
            j = idx[idx != i]
            life = max(en[i] - st[i], 1e-9)
            out[i] = np.clip(np.minimum(en[i], oen[j]) - np.maximum(st[i], ost[j]), 0, None).sum() / life
    return out


def _has_shared_first_block(fin):
    tabs = fin.block_tables.cpu().numpy()
    lens = fin.context_lens.cpu().numpy()
    # the kernel looks for shared prefixes in batches of 2..64 rows
    return 2 <= len(lens) <= 64 and any(lens[i] > 16 and lens[i - 1] > 16 and tabs[i, 0] == tabs[i - 1, 0]
               for i in range(1, len(lens)))


def varlen(name, trace):
    w, r, fin, pools = _prepare(name)

    def call(i):
        kc, vc = pools[i % POOLS]
        pa.varlen(fin.q, fin.query_start_loc, fin.context_lens, kc, vc, fin.block_tables,
                  w.scale, fin.out, fin.max_query_len, fin.max_context_len, fin.workspace,
                  kv_scales=r.kv_scales, layout=pa.LAYOUT_ROTATED)

    for raw in _record(call, trace):
        d = raw[VARLEN_OFFSET:].reshape(-1, 4)
        d = d[d[:, 0] > 0]
        t0 = d[:, 0].min()
        st, en = (d[:, 0] - t0) / 100.0, (d[:, 1] - t0) / 100.0
        kind = (d[:, 2] >> 62) & 3
        tiles = (d[:, 2] & 0xFFFF).astype(float)
        pf, dc = kind == 1, kind == 2
        print(f"== {name}: span {en.max():.1f} us; {pf.sum()} prefill and {dc.sum()} decode workgroups")
        if pf.any():
            per = (en[pf] - st[pf]) / np.maximum(tiles[pf], 1)
            big = pf & (tiles >= _pct(tiles[pf], 90))
            print(f"   prefill: tiles med {np.median(tiles[pf]):.0f} max {tiles[pf].max():.0f}; "
                  f"us per tile med {np.median(per):.2f} (units with the most tiles "
                  f"{np.median((en[big] - st[big]) / tiles[big]):.2f}); ends: "
                  + ", ".join(f"{q}% by {_pct(en[pf], q):.1f}" for q in (25, 50, 75, 90, 100)))
            # the units with the most tiles: how much of their life they had
            # their CU to themselves (HW_ID: CU, SH, SE; with the XCC)
            cu = _cu_ids(d[:, 3] & 0xF, (d[:, 3] >> 32).astype(np.int64))
            alone = 1 - _peers(cu, st, en, st, en)[big]
            bt = (en[big] - st[big]) / tiles[big]
            lone = alone > np.median(alone)
            print(f"   units with the most tiles: alone on their CU for {np.median(alone):.2f} of their "
                  f"life (median); us per tile {np.median(bt[lone]):.2f} for the more alone half, "
                  f"{np.median(bt[~lone]):.2f} for the other")
        if dc.any():
            dur = en[dc] - st[dc]
            print(f"   decode: starts " + ", ".join(f"{q}% by {_pct(st[dc], q):.1f}" for q in (10, 50, 90))
                  + f"; duration med {np.median(dur):.1f} p90 {_pct(dur, 90):.1f}; last ends {en[dc].max():.1f}")
        print("   running (prefill / decode workgroups): " + ", ".join(
            f"t={t}: {((st[pf] <= t) & (en[pf] > t)).sum()}/{((st[dc] <= t) & (en[dc] > t)).sum()}"
            for t in range(0, int(en.max()) + 1, 20)))


def main(argv):
    if len(argv) < 2 or argv[0] not in ("decode", "varlen"):
        raise SystemExit(__doc__)
    _load()
    if not hasattr(pa._lib, "pa_trace_set"):
        raise SystemExit(f"{pa.LIB_PATH} is not a timeline build")
    import runpy
    digest = runpy.run_path(os.path.join(_HERE, "build.py"))["sources_digest"]()
    stamp = pa.LIB_PATH + ".sources"
    if not os.path.exists(stamp) or open(stamp).read().strip() != digest:
        raise SystemExit(f"{pa.LIB_PATH} was built from other sources: rebuild it "
                         f"(python {os.path.join(_HERE, 'build.py')} --timeline)")
    pa._lib.pa_trace_set.argtypes = [ctypes.c_void_p]
    trace = torch.zeros(TRACE_STAMPS, dtype=torch.int64, device="cuda")
    for name in argv[1:]:
        (decode if argv[0] == "decode" else varlen)(name, trace)
        sys.stdout.flush()


if __name__ == "__main__":
    main(sys.argv[1:])
