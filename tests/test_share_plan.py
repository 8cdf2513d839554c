"""Host model of the decode plan with shared prefixes (no GPU).

When consecutive decode rows start on the same physical block, the plan of
the matrix-core decode kernel groups them (runs cut into groups of 16 / G
rows) and lays out, per KV head, a line of items: the group's shared item
(its common leading chunks, attended once for all of the group's query
heads) before the first row's own item, then the own items of the other
rows.  The line is cut into W equal ranges as for plain rows.

This model restates those rules and checks what the kernels rely on, over
random and adversarial batches: every chunk of every item is processed by
exactly one wave; a wave's shared segments and own segments get partial
indices (wave + group, wave + row) that never collide and stay inside the
workspace regions sized by the library; every row gets exactly one plan
entry and one shared-plan entry, and the merge's reads land on partials
that some wave wrote; a wave's segment list and table entries fit its LDS
area; the chunk count of a wave is zero exactly when it has no segment;
and the shared tokens of a group are a chunk multiple below every member's
last token.  The workspace sizes come from the library itself.
"""
import numpy as np
import pytest

from tests.libutil import ensure_built

CHUNK, Q, BETA, SEG_INTS, LDS_INTS = 16, 8, 32, 8, 2048


def plan_max_cost(block):
    m = CHUNK // block if CHUNK > block else 1
    x = LDS_INTS - SEG_INTS - m
    return 1 + min(x * (Q + BETA) // (SEG_INTS + m), x * Q // m)


def launch_waves(rows, max_ctx, block, hkv):
    cmax = -(-max_ctx // CHUNK)
    tmax = rows * (BETA + Q * cmax)
    w = max(-(-tmax // plan_max_cost(block)), 1024 // hkv)
    return min(w, rows * max(1, cmax))


def plan(tabs, ctx, G, block, hkv):
    """The device plan, restated: per row (L, n, S, group number) and the
    items' costs, then the segments of every wave."""
    rows = len(ctx)
    M = 16 // G
    c = list(ctx) + [-1] * (64 - rows)
    cand, s_pair, lims = [False] * 64, [0] * 64, [0] * 64
    for r in range(1, 64):
        lims[r] = min(c[r], c[r - 1]) - 1
        if c[r] > 0 and c[r - 1] > 0 and lims[r] >= CHUNK and tabs[r][0] == tabs[r - 1][0]:
            cand[r] = True
    # 15 probes at equal steps over the blocks of the longest candidate
    # pair's common tokens, the same positions for every pair; a pair
    # compares those inside its own common blocks
    nbk = -(-max([lims[r] for r in range(64) if cand[r]], default=0) // block)
    for r in range(1, 64):
        if cand[r]:
            lim_b = -(-lims[r] // block)
            lcp, run = 1, True
            for k in range(1, 16):
                pos = k * (nbk - 1) // 15
                run = run and pos < lim_b and tabs[r][pos] == tabs[r - 1][pos]
                if run:
                    lcp = pos + 1
            s_pair[r] = min(lcp * block, lims[r])
    grp = []
    for r in range(64):
        run0 = max(i for i in range(r + 1) if not cand[i])
        L = r - (r - run0) % M
        more, i = 0, L + 1
        while i < 64 and cand[i]:
            more, i = more + 1, i + 1
        n = 1 + min(M - 1, more)
        smin = min([s_pair[L + m] for m in range(1, n)], default=0)
        S = smin // CHUNK * CHUNK if n >= 2 else 0
        grp.append((L, n, S if S >= CHUNK else 0))
    if not any(cand):  # the plain split
        grp = [(r, 1, 0) for r in range(64)]
    lead = [g[2] > 0 and g[0] == r for r, g in enumerate(grp)]
    gnum = list(np.cumsum([0] + lead)[:64])
    items = []  # (row, kind, first unit, chunks, first token)
    x = 0
    for r in range(64):
        L, n, S = grp[r]
        if lead[r]:
            items.append((r, "sh", x, S // CHUNK, 0))
            x += BETA + Q * (S // CHUNK)
        if c[r] < 0:
            continue
        tok = S if S > 0 else 0
        cp = -(-(c[r] - tok) // CHUNK) if c[r] > tok else 0
        if S > 0 and cp == 0:
            continue
        items.append((r, "pr", x, cp, tok))
        x += BETA + Q * cp
    T = x
    W = min(max(-(-T // plan_max_cost(block)), 1024 // hkv),
            launch_waves(rows, max(ctx), block, hkv), max(1, T // Q))
    waves = []
    for y in range(W):
        lo, hi = y * T // W, (y + 1) * T // W
        segs = []
        for r, kind, x0, cc, tok in items:
            x1 = x0 + BETA
            jl = -(-(lo - x1) // Q) if lo > x1 else 0
            jh = min(cc, -(-(hi - x1) // Q)) if hi > x1 else 0
            if jl < jh:
                segs.append((r, kind, jl, jh, tok))
        waves.append(segs)
    return grp, lead, gnum, items, T, W, waves


def check(tabs, ctx, G, block, hkv, ws_bytes):
    rows = len(ctx)
    grp, lead, gnum, items, T, W, waves = plan(tabs, ctx, G, block, hkv)
    parts = launch_waves(rows, max(ctx), block, hkv)
    H = hkv * G
    # workspace regions the library sized: own (parts + rows) x H columns,
    # shared (parts + rows // 2) x hkv x 16 columns, head dim 128
    own_cols, sh_cols = (parts + rows) * H, (parts + rows // 2) * hkv * 16
    plan4 = (2 * rows + 3) // 4 * 4
    need = 4 * (2 * plan4 + own_cols * 130 + sh_cols * 130)
    assert ws_bytes == need
    for r in range(rows):
        L, n, S = grp[r]
        if S:
            assert S % CHUNK == 0 and S <= ctx[r] - 1
            assert all(tabs[L + m][0] == tabs[L][0] for m in range(n))
    covered = {}
    own_idx, sh_idx = set(), set()
    for y, segs in enumerate(waves):
        K = sum(jh - jl for _, _, jl, jh, _ in segs)
        assert (K == 0) == (len(segs) == 0)
        ents = 0
        for r, kind, jl, jh, tok in segs:
            c0 = tok // CHUNK
            ents += ((c0 + jh) * CHUNK - 1) // block - ((c0 + jl) * CHUNK) // block + 1
            for j in range(jl, jh):
                key = (r, kind, j)
                assert key not in covered
                covered[key] = y
            if kind == "sh":
                idx = y + gnum[r]
                assert (idx,) not in sh_idx and idx < parts + rows // 2
                sh_idx.add((idx,))
            else:
                idx = y + r
                assert idx not in own_idx and idx < parts + rows
                own_idx.add(idx)
        assert len(segs) * SEG_INTS + ents <= LDS_INTS
    for r, kind, x0, cc, tok in items:
        for j in range(cc):
            assert (r, kind, j) in covered
        # a row's pieces sit on consecutive waves (the merge reads a range)
        ys = sorted({covered[(r, kind, j)] for j in range(cc)})
        assert ys == list(range(ys[0], ys[-1] + 1)) if ys else True


def _tables(rng, spec, nb, block):
    free = list(rng.permutation(nb))
    width = max(-(-cx // block) for cx, _ in spec) or 1
    tabs = np.full((64, width), -1, np.int64)
    for r, (cx, share) in enumerate(spec):
        for i in range(-(-cx // block)):
            tabs[r, i] = tabs[share[0], i] if share is not None and i < share[1] else free.pop()
    return tabs


def _spec(rng, rows, block):
    spec = []
    while len(spec) < rows:
        kind = rng.integers(0, 4)
        prompt = int(rng.integers(0, 3000))
        if kind == 0 or prompt < block:
            spec.append((int(rng.integers(0, 2000)), None))
            continue
        lead = len(spec)
        spec.append((prompt + int(rng.integers(1, 300)), None))
        for _ in range(int(rng.integers(1, 8))):
            if len(spec) >= rows:
                break
            nb = -(-prompt // block) if rng.random() < 0.7 else int(rng.integers(1, -(-prompt // block) + 1))
            spec.append((prompt + int(rng.integers(1, 300)), (lead, nb)))
    return spec[:rows]


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("block", [4, 16, 64])
def test_shared_plan_invariants(G, block):
    ensure_built()
    import paged_kv_cache_158_amd as pa
    rng = np.random.default_rng(G * 100 + block)
    for trial in range(12):
        rows = int(rng.integers(2, 65))
        hkv = int(rng.choice([1, 2, 8]))
        spec = _spec(rng, rows, block)
        ctx = [cx for cx, _ in spec]
        if max(ctx) == 0:
            continue
        nb = sum(-(-cx // block) for cx in ctx) + 8
        tabs = _tables(rng, spec, nb, block)
        d = pa.CacheDims(num_blocks=nb, block_size=block, num_heads=hkv * G, num_kv_heads=hkv,
                         head_dim=128, dtype=pa.DTYPE_BF16)
        check(tabs, ctx, G, block, hkv, pa.decode_workspace_bytes(d, rows, max(ctx)))


def test_groups_of_the_fork_workload_shape():
    # 16 groups of 4 forks of a 1024-token prompt (G = 4): 16 shared items of
    # about 1024 tokens, every row's own item holds its suffix
    rng = np.random.default_rng(1)
    spec = []
    for _ in range(16):
        lead = len(spec)
        spec.append((1024 + int(rng.integers(1, 257)), None))
        spec += [(1024 + int(rng.integers(1, 257)), (lead, 64)) for _ in range(3)]
    tabs = _tables(rng, spec, 4096, 16)
    ctx = [cx for cx, _ in spec]
    grp, lead, *_ = plan(tabs, ctx, 4, 16, 8)
    assert sum(lead) == 16
    step = (-(-(max(ctx) - 1) // 16) - 1) // 15 + 1  # blocks between probes, at most
    for r in range(0, 64, 4):
        L, n, S = grp[r]
        assert (L, n) == (r, 4) and 1024 - step * 16 <= S <= 1024
