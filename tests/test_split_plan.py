"""Host model of the balanced decode split (no GPU).

The decode kernel splits the work of each KV head as follows: active row r
costs ROW + CHUNK * c_r units on a line (c_r = chunks of its context), the
line of length T is cut into W equal ranges, and wave y processes the chunks
whose first unit lies in [floor(y T / W), floor((y+1) T / W)).  W is at
least 1024 / H_kv, large enough that every range fits RMAX units (the bound
that keeps a wave's segment list and block-table entries inside its 8 KiB
of LDS), at most the launch's waves and at most T / CHUNK.

This model checks the properties the kernel relies on, over adversarial
length mixes: every chunk is processed exactly once, a row's segments sit
on consecutive waves starting at the wave the kernel computes from the
row's first chunk, partial indices (wave + row) never collide, and the LDS
bound holds.  The launch size comes from the library's own workspace size,
so a change of the split constants in the library shows up here.
"""
import numpy as np
import pytest

from tests.libutil import ensure_built

CHUNK_COST, ROW_COST = 8, 32
LDS_INTS, SEG_INTS = 2048, 8


def rmax(chunk, block):
    m = chunk // block if chunk > block else 1
    x = LDS_INTS - SEG_INTS - m
    return 1 + min(x * (CHUNK_COST + ROW_COST) // (SEG_INTS + m), x * CHUNK_COST // m)


def grid_waves(rows, max_ctx, chunk, block, share):
    cmax = -(-max_ctx // chunk)
    tmax = rows * (ROW_COST + CHUNK_COST * cmax)
    w = max(-(-tmax // rmax(chunk, block)), share)
    return min(w, rows * max(1, cmax))


def split(ctx, chunk, block, share, launch):
    """Segments (row, first chunk, end chunk) of every wave, and W."""
    c = [-(-x // chunk) for x in ctx]
    first = np.concatenate([[0], np.cumsum([ROW_COST + CHUNK_COST * ci for ci in c])])
    T = int(first[-1])
    W = max(-(-T // rmax(chunk, block)), share)
    W = min(W, launch, max(1, T // CHUNK_COST))
    waves = []
    for y in range(W):
        lo, hi = y * T // W, (y + 1) * T // W
        segs = []
        for r, cr in enumerate(c):
            x0 = int(first[r]) + ROW_COST
            jl = -(-(lo - x0) // CHUNK_COST) if lo > x0 else 0
            jh = min(cr, -(-(hi - x0) // CHUNK_COST)) if hi > x0 else 0
            if jl < jh:
                segs.append((r, jl, jh))
        waves.append(segs)
    return waves, W, T, first, c


def check(ctx, chunk, block, share, launch):
    waves, W, T, first, c = split(ctx, chunk, block, share, launch)
    lb = int(np.log2(block))
    used = set()
    for y, segs in enumerate(waves):
        entries = sum(((jh * chunk - 1) >> lb) - ((jl * chunk) >> lb) + 1 for _, jl, jh in segs)
        assert SEG_INTS * len(segs) + entries <= LDS_INTS, (y, len(segs), entries)
        for r, _, _ in segs:
            assert (y + r) not in used
            used.add(y + r)
    assert max(y + r for y, s in enumerate(waves) for r, _, _ in s) < launch + len(ctx)
    for r, cr in enumerate(c):
        got = [(jl, jh, y) for y, s in enumerate(waves) for (rr, jl, jh) in s if rr == r]
        pos = 0
        for jl, jh, _ in got:
            assert jl == pos
            pos = jh
        assert pos == cr
        if cr:
            ys = [y for _, _, y in got]
            assert ys == list(range(ys[0], ys[0] + len(ys)))
            x0 = int(first[r]) + ROW_COST
            wave_of = lambda x: ((x + 1) * W - 1) // T
            assert ys[0] == wave_of(x0) and ys[-1] == wave_of(x0 + CHUNK_COST * (cr - 1))
    return W


def test_model_matches_library_launch_size():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    d = pa.CacheDims(num_blocks=16, block_size=16, num_heads=32, num_kv_heads=8, head_dim=128,
                     dtype=pa.DTYPE_BF16)
    for rows, ctx in [(32, 2048), (3, 40000), (1000, 20000), (200, 100000), (7, 9), (1, 300)]:
        plan = (2 * rows + 3) // 4 * 4
        floats = pa.decode_workspace_bytes(d, rows, ctx) // 4 - plan
        if 2 <= rows <= 64:
            # shared-prefix region: plan, then 16 columns per KV head for
            # (waves + rows // 2) shared partial indices
            floats -= plan + (rows // 2) * 8 * 16 * 130
            waves, rest = divmod(floats - rows * 32 * 130, 32 * 130 + 8 * 16 * 130)
        else:
            waves, rest = divmod(floats - rows * 32 * 130, 32 * 130)
        assert rest == 0
        assert waves == grid_waves(rows, ctx, 16, 16, 128), (rows, ctx)


@pytest.mark.parametrize("kind", range(4))
def test_split_covers_every_chunk_once_within_lds(kind):
    rng = np.random.default_rng(100 + kind)
    for trial in range(60):
        chunk = int(rng.choice([8, 16, 32]))
        block = int(rng.choice([4, 8, 16, 32, 256]))
        rows = int(rng.integers(1, 160))
        if kind == 0:
            ctx = rng.integers(0, 3000, rows)
        elif kind == 1:  # tiny and empty rows
            ctx = rng.integers(0, 3, rows)
        elif kind == 2:  # a few huge rows among short ones
            ctx = np.where(rng.random(rows) < 0.05, rng.integers(50000, 200000, rows),
                           rng.integers(1, 40, rows))
        else:
            ctx = rng.integers(0, 100000, rows)
        ctx = [int(x) for x in ctx]
        share = int(rng.choice([64, 128, 1024]))
        launch = grid_waves(rows, max(ctx), chunk, block, share)
        check(ctx, chunk, block, share, launch)
