"""GPU parity of decode batches whose rows share leading blocks.

Rows that start on the same physical blocks (parallel sampling and beam
search after copy-on-write forks, prefix-cache hits; vLLM docs page,
写时复制 and Prefix Caching; SourceAIX page §5.2.1) have their common prefix
attended once for all of their query heads.  These tests build block tables
directly (not through the block manager) so that the sharing takes every
form the kernels must handle: groups cut from long runs of sharing rows,
rows whose whole context is shared, empty rows between groups, and tables
that agree at the entries the plan probes but differ between them (the
staged-table check then sends those chunks through each row's own blocks).
Every output is held to the bf16 bar against the fp64 oracle, which reads
each row through its own table.
"""
import numpy as np
import pytest

import synth
from oracle import attention
from tests.libutil import LAYOUT_PLAIN, LAYOUT_ROTATED, ensure_built
from tests.test_gpu_decode import check_out

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()


B, D, HKV = 16, 128, 2


def _probes(lim):
    """Table positions the plan compares when the longest pair of rows that
    may share tokens shares at most lim: entry 0 and 15 more at equal steps
    over those blocks (a pair compares the ones inside its own common
    blocks)."""
    nb = -(-lim // B)
    return {k * (nb - 1) // 15 for k in range(16)}


def _tables(rng, spec, nb):
    """Block tables from a spec of rows: each row is (ctx, share) where
    share = (row it copies from, blocks copied) or None.  Blocks not copied
    are fresh, distinct draws from the pool."""
    free = list(rng.permutation(nb))
    width = max(-(-c // B) for c, _ in spec) or 1
    tabs = np.full((len(spec), width), -1, np.int32)
    for r, (ctx, share) in enumerate(spec):
        n = -(-ctx // B)
        for i in range(n):
            if share is not None and i < share[1]:
                tabs[r, i] = tabs[share[0], i]
            else:
                tabs[r, i] = free.pop()
    return tabs


def _run(spec, G, dtype="bf16", seed=0, tabs=None, layout=LAYOUT_PLAIN, nb=1024, ren=None):
    """Decode of the batch on the GPU against the oracle; with `ren`, every
    physical block b is renamed ren[b] (pool rows moved, tables rewritten)
    before the GPU call, which must not change a single output bit."""
    import paged_kv_cache_158_amd as pa
    from paged_kv_cache_158_amd import engine
    H = HKV * G
    ctx = np.array([c for c, _ in spec], np.int32)
    if tabs is None:
        tabs = _tables(np.random.default_rng(seed + 1000), spec, nb)
    rng = np.random.default_rng(seed)  # q and the pool, whatever the tables
    n = len(spec)
    q = synth.f32_to_bf16_bits(rng.normal(0, 1, (n, H, D)).astype(np.float32))
    if dtype == "fp8":
        kc = rng.integers(0, 0x7E, (nb, B, HKV, D)).astype(np.uint8) | (
            rng.integers(0, 2, (nb, B, HKV, D)).astype(np.uint8) << 7)
        vc = rng.integers(0, 0x7E, (nb, B, HKV, D)).astype(np.uint8) | (
            rng.integers(0, 2, (nb, B, HKV, D)).astype(np.uint8) << 7)
        ks = rng.uniform(3.5, 5, HKV).astype(np.float32) / 448
        vs = rng.uniform(3.5, 5, HKV).astype(np.float32) / 448
    else:
        kc = synth.f32_to_bf16_bits(rng.normal(0, 1, (nb, B, HKV, D)).astype(np.float32))
        vc = synth.f32_to_bf16_bits(rng.normal(0, 1, (nb, B, HKV, D)).astype(np.float32))
    scale = 1.0 / np.sqrt(D)
    gtabs = tabs
    gkc, gvc = kc, vc
    if ren is not None:
        gtabs = np.where(tabs >= 0, ren[np.maximum(tabs, 0)], -1).astype(np.int32)
        gkc, gvc = np.empty_like(kc), np.empty_like(vc)
        gkc[ren], gvc[ren] = kc, vc
    # device caches in the requested head order
    perm = np.array([[pa.cache_head_index(h, p, HKV, layout) for h in range(HKV)]
                     for p in range(B)])
    def phys(x):
        out = np.empty_like(x)
        for p in range(B):
            out[:, p, perm[p], :] = x[:, p, :, :]
        return out
    if dtype == "fp8":
        gk = torch.from_numpy(phys(gkc)).cuda().view(torch.float8_e4m3fn)
        gv = torch.from_numpy(phys(gvc)).cuda().view(torch.float8_e4m3fn)
        sc = (torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda())
    else:
        gk = engine.to_device(phys(gkc), "bf16", "cuda")
        gv = engine.to_device(phys(gvc), "bf16", "cuda")
        sc = None
    gq = engine.to_device(q, "bf16", "cuda")
    out = torch.empty_like(gq)
    gt = torch.from_numpy(gtabs).cuda()
    gc = torch.from_numpy(ctx).cuda()
    pa.decode(gq, gk, gv, gt, gc, scale, out, int(ctx.max()), 0, kv_scales=sc, layout=layout)
    torch.cuda.synchronize()
    if dtype == "fp8":
        ref = attention.decode(q, kc, vc, tabs, ctx, scale, "bf16", HKV, cache_dtype="fp8",
                               k_scale=ks, v_scale=vs)
    else:
        ref = attention.decode(q, kc, vc, tabs, ctx, scale, "bf16", HKV)
    got = engine.to_host_bits(out)
    check_out(got, ref, "bf16", f"shared prefix G{G} {dtype}")
    return got, tabs


def _groups(rng, n_groups, per, prompt, suffix_hi):
    spec = []
    for _ in range(n_groups):
        lead = len(spec)
        spec.append((prompt + int(rng.integers(1, suffix_hi)), None))
        for _ in range(per - 1):
            spec.append((prompt + int(rng.integers(1, suffix_hi)), (lead, prompt // B)))
    return spec


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fork_groups(G, dtype):
    # groups of 4 rows sharing a 640-token prompt, private suffixes
    spec = _groups(np.random.default_rng(1), 6, 4, 640, 200)
    _run(spec, G, dtype, seed=2)


@pytest.mark.parametrize("G", [4, 8])
def test_long_runs_cut_into_groups(G):
    # 7 rows sharing one prompt (groups of 16 / G rows), then a lone row,
    # then 3 sharing rows whose common part varies, an empty row, a short row
    spec = [(900, None)] + [(900 + 37 * i, (0, 50)) for i in range(1, 7)]
    spec += [(333, None)]
    spec += [(700, None), (650, (8, 30)), (800, (8, 20))]
    spec += [(0, None), (9, None)]
    _run(spec, G, seed=3)


def test_whole_context_shared():
    # identical rows: everything but each row's last token is attended once
    # (a row's last token is never shared), contexts a chunk multiple and not
    spec = [(512, None), (512, (0, 32)), (512, (0, 32)), (512, (0, 32)), (496, (0, 31))]
    _run(spec, 4, seed=4)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [4, 8])
def test_tables_differing_between_probes(dtype, G):
    # rows 1-3 copy row 0's table at the probed positions only: every other
    # entry is a block of their own, so most shared chunks differ
    rng = np.random.default_rng(5)
    ctx = 1000
    spec = [(ctx, None)] + [(ctx, (0, -(-ctx // B))) for _ in range(3)]
    tabs = _tables(rng, spec, 1024)
    keep = _probes(ctx - 1)  # a row's last token is never shared
    free = [b for b in rng.permutation(1024) if b not in set(tabs.ravel())]
    for r in range(1, 4):
        for i in range(tabs.shape[1]):
            if i not in keep:
                tabs[r, i] = free.pop()
    _run(spec, G, dtype, seed=6, tabs=tabs)


def test_rotated_layout_and_relabelling():
    spec = _groups(np.random.default_rng(7), 4, 4, 480, 90)
    got, tabs = _run(spec, 4, seed=8, layout=LAYOUT_ROTATED)
    ren = np.random.default_rng(9).permutation(1024).astype(np.int32)
    got2, _ = _run(spec, 4, seed=8, tabs=tabs, layout=LAYOUT_ROTATED, ren=ren)
    assert (got == got2).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_ranges_not_a_multiple_of_the_workgroup(dtype):
    # 3 rows of 7 chunks make 21 ranges per KV head: bf16 workgroups hold
    # four waves, so the last one has three waves with no range, which still
    # take part in the probe exchange before they leave
    spec = [(100, None), (104, (0, 6)), (110, (0, 6))]
    _run(spec, 4, dtype, seed=13)


def test_max_rows_and_beyond():
    # 64 rows (the largest batch that looks for sharing) and 65 (none)
    rng = np.random.default_rng(10)
    for n_groups in (16,):
        spec = _groups(rng, n_groups, 4, 256, 60)
        _run(spec, 4, seed=11)
        _run(spec + [(100, None)], 4, seed=12)
