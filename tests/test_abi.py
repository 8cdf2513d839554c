"""The C-ABI library loads, exports every symbol include/pa.h declares, and
rejects bad arguments on the host before anything reaches a GPU."""
import ctypes
import os
import re

import pytest

from tests.libutil import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    lib = pa._lib
    syms = declared_symbols()
    assert "pa_decode" in syms and "pa_cache_write" in syms and "pa_bm_append" in syms
    missing = [s for s in syms if not hasattr(lib, s)]
    assert not missing, missing


def test_timeline_build_has_the_same_abi_and_the_product_none_of_it():
    # libpa_timeline.so (build.py --timeline) is the same sources with
    # per-wave timestamps: every declared entry point plus pa_trace_set; the
    # product library exports no trace entry point
    ensure_built()
    import paged_kv_cache_158_amd as pa
    assert not hasattr(pa._lib, "pa_trace_set")
    path = os.path.join(os.path.dirname(pa.__file__), "libpa_timeline.so")
    if not os.path.exists(path):
        pytest.skip("timeline build not present (python paged_kv_cache_158_amd/build.py --timeline)")
    tl = ctypes.CDLL(path)
    missing = [s for s in declared_symbols() + ["pa_trace_set"] if not hasattr(tl, s)]
    assert not missing, missing


def test_single_hip_runtime_in_process():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    assert len(pa._hip_runtimes()) == 1


def test_status_strings_and_version():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    assert pa.version() >= 100
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert pa.status_string(st) and pa.status_string(st) != "unknown status"


def _dims(pa, **kw):
    d = dict(num_blocks=16, block_size=16, num_heads=32, num_kv_heads=8, head_dim=128,
             dtype=pa.DTYPE_BF16)
    d.update(kw)
    return pa.CacheDims(**d)


def test_host_validation_rejects_before_launch():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    L = pa._lib
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    d = _dims(pa)
    # null pointers
    assert L.pa_cache_write(None, fake, fake, 4, fake, fake, ctypes.byref(d), None) == pa.PA_ERR_INVALID_ARG
    # misaligned pointer
    assert L.pa_cache_write(ctypes.c_void_p(0x1002), fake, fake, 4, fake, fake, ctypes.byref(d),
                            None) == pa.PA_ERR_INVALID_ARG
    # unsupported shapes
    for bad in (dict(head_dim=96), dict(block_size=12), dict(block_size=2), dict(dtype=7)):
        db = _dims(pa, **bad)
        assert L.pa_cache_write(fake, fake, fake, 4, fake, fake, ctypes.byref(db), None) == \
            pa.PA_ERR_UNSUPPORTED, bad
    db = _dims(pa, num_heads=30)
    assert L.pa_cache_write(fake, fake, fake, 4, fake, fake, ctypes.byref(db), None) == \
        pa.PA_ERR_INVALID_ARG
    # zero tokens / pairs / sequences are no-ops that touch nothing
    assert L.pa_cache_write(None, None, None, 0, None, None, ctypes.byref(d), None) == pa.PA_OK
    assert L.pa_copy_blocks(None, None, None, 0, ctypes.byref(d), None) == pa.PA_OK
    assert L.pa_swap_blocks(None, None, 4, None, None, 4, None, 0, ctypes.byref(d), None) == pa.PA_OK
    # swap pools must be device or pinned host memory: plain host memory (and
    # null, and bad counts) is refused before anything is launched
    import numpy as np
    host = np.zeros(1 << 16, dtype=np.uint8)
    hp = ctypes.c_void_p(host.ctypes.data)
    assert L.pa_swap_blocks(hp, hp, 4, hp, hp, 4, hp, 1, ctypes.byref(d), None) == \
        pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks(None, hp, 4, hp, hp, 4, hp, 1, ctypes.byref(d), None) == \
        pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks(hp, hp, 0, hp, hp, 4, hp, 1, ctypes.byref(d), None) == \
        pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks(hp, hp, 4, hp, hp, 4, hp, -1, ctypes.byref(d), None) == \
        pa.PA_ERR_INVALID_ARG
    dec = pa._decode
    assert dec(None, None, None, None, 0, None, 0, 0, 1.0, None, ctypes.byref(d), 0, None, 0,
               None) == pa.PA_OK
    # group 3 is not built
    d3 = _dims(pa, num_heads=24)
    assert dec(fake, fake, fake, fake, 4, fake, 2, 64, 1.0, fake, ctypes.byref(d3), 0, None, 0,
               None) == pa.PA_ERR_UNSUPPORTED
    # workspace needed but missing / too small
    need = pa.decode_workspace_bytes(d, 4, 4096, 512)
    assert need > 0
    assert dec(fake, fake, fake, fake, 256, fake, 4, 4096, 1.0, fake, ctypes.byref(d), 512, None,
               0, None) == pa.PA_ERR_WORKSPACE
    assert dec(fake, fake, fake, fake, 256, fake, 4, 4096, 1.0, fake, ctypes.byref(d), 512, fake,
               need - 16, None) == pa.PA_ERR_WORKSPACE
    # partition size must be a multiple of 64
    assert dec(fake, fake, fake, fake, 256, fake, 4, 4096, 1.0, fake, ctypes.byref(d), 100, fake,
               1 << 30, None) == pa.PA_ERR_INVALID_ARG


def test_partition_and_workspace_sizes():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    d = _dims(pa)
    # library choice: the balanced per-row split (0) while the rows fit one plan
    assert pa.decode_partition_size(d, 8, 32768) == 0
    assert pa.decode_partition_size(d, 32, 2048) == 0
    assert pa.decode_partition_size(d, 1, 100) == 0
    assert pa.decode_partition_size(d, 1024, 4096) == 0
    # beyond 1024 rows: the largest fixed partition giving >= 1024 waves
    assert pa.decode_partition_size(d, 1025, 4096) == 2048
    assert pa.decode_partition_size(d, 4, 4096, 192) == 192
    # balanced workspace: plan (rows x 2 int32), then (m, l) and o for every
    # (partial, query head), partial index = wave + row < waves + rows.
    # waves per KV head = max(1024 / H_kv, ceil(longest line / 9063)), the
    # line being rows x (32 + 8 ceil(ctx / 16)) cost units and 9063 the
    # longest range whose segment list and block-table entries fit 8 KiB
    def waves(rows, ctx):
        line = rows * (32 + 8 * -(-ctx // 16))
        return max(128, -(-line // 9063))
    assert waves(32, 2048) == 128 and waves(1000, 20000) == 1107
    # 2..64 rows (4 query heads per KV head here) add the shared-prefix
    # region: a second plan (rows x 2), then (m, l) and o for 16 query
    # columns per KV head and shared partial index wave + group < waves +
    # rows / 2
    for rows, ctx in [(32, 2048), (3, 40000), (1000, 20000), (1, 5000), (64, 100), (65, 100)]:
        pairs = (waves(rows, ctx) + rows) * 32
        plan = (2 * rows + 3) // 4 * 4
        need = plan + pairs * 2 + pairs * 128
        if 2 <= rows <= 64:
            cols = (waves(rows, ctx) + rows // 2) * 8 * 16
            need += plan + cols * 2 + cols * 128
        assert pa.decode_workspace_bytes(d, rows, ctx) == 4 * need, (rows, ctx)
    # no workspace when every context fits one partition
    assert pa.decode_workspace_bytes(d, 32, 512, 512) == 0
    parts = 64
    rows = 8 * 32 * parts
    assert pa.decode_workspace_bytes(d, 8, 32768, 512) == 4 * ((rows * 2 + 3) // 4 * 4 + rows * 128)


def test_cache_head_index_both_layouts():
    ensure_built()
    import paged_kv_cache_158_amd as pa
    # plain: head h at index h; rotated (power-of-two heads): (h + p) mod H
    for hkv in (1, 2, 4, 8, 16):
        for p in range(0, 40, 3):
            idx_plain = [pa.cache_head_index(h, p, hkv, pa.LAYOUT_PLAIN) for h in range(hkv)]
            idx_rot = [pa.cache_head_index(h, p, hkv, pa.LAYOUT_ROTATED) for h in range(hkv)]
            assert idx_plain == list(range(hkv))
            assert idx_rot == [(h + p) % hkv for h in range(hkv)]
    # not a power of two: no rotation
    assert [pa.cache_head_index(h, 5, 3, pa.LAYOUT_ROTATED) for h in range(3)] == [0, 1, 2]
    # out of range
    assert pa.cache_head_index(4, 0, 4, pa.LAYOUT_PLAIN) == -1
    assert pa.cache_head_index(-1, 0, 4, pa.LAYOUT_PLAIN) == -1
    assert pa.cache_head_index(0, -1, 4, pa.LAYOUT_ROTATED) == -1
    assert pa.cache_head_index(0, 0, 4, 7) == -1
    # an unknown layout in the dims is refused before any launch
    fake = ctypes.c_void_p(0x1000)
    d = _dims(pa, layout=5)
    assert pa._lib.pa_cache_write(fake, fake, fake, 4, fake, fake, ctypes.byref(d), None) == \
        pa.PA_ERR_UNSUPPORTED


def test_varlen_checks_every_kernel_it_may_need_before_launching():
    # bf16, head_dim 64, 16 query heads per KV head: the prefill kernel
    # exists, the decode kernel (which one-row segments need) does not, so
    # the call is refused whole, before anything is launched
    ensure_built()
    import paged_kv_cache_158_amd as pa
    fake = ctypes.c_void_p(0x1000)
    d = _dims(pa, num_heads=32, num_kv_heads=2, head_dim=64)
    st = pa._varlen(fake, fake, fake, 2, 64, 63, 128, fake, fake, fake, 8, 1.0, fake,
                    ctypes.byref(d), fake, 1 << 30, None)
    assert st == pa.PA_ERR_UNSUPPORTED


def test_varlen_refuses_blocks_beyond_32_bit_offsets():
    # the prefill kernels address one cache block with 32-bit byte offsets:
    # 256 tokens x 65537 KV heads x 128 dims x 2 bytes is past 4 GiB, so the
    # call is refused before anything is launched
    ensure_built()
    import paged_kv_cache_158_amd as pa
    fake = ctypes.c_void_p(0x1000)
    d = _dims(pa, num_blocks=8, block_size=256, num_heads=4 * 65537, num_kv_heads=65537)
    st = pa._varlen(fake, fake, fake, 2, 64, 63, 128, fake, fake, fake, 8, 1.0, fake,
                    ctypes.byref(d), fake, 1 << 30, None)
    assert st == pa.PA_ERR_UNSUPPORTED


def test_varlen_workspace_depends_on_the_arguments_only():
    # sized without any device query (this runs with no GPU): a lone long
    # chunk gets the cut pieces' partials on top of the decode layout
    ensure_built()
    import paged_kv_cache_158_amd as pa
    d = _dims(pa, num_blocks=4096)
    decode_only = pa.decode_workspace_bytes(d, 1, 32768, 0)
    with_cut = pa.varlen_workspace_bytes(d, 1, 512, 512, 32768)
    assert with_cut > decode_only
    assert with_cut == pa.varlen_workspace_bytes(d, 1, 512, 512, 32768)
    # many units per KV head: no cut, no extra bytes
    assert pa.varlen_workspace_bytes(d, 128, 2172, 512, 4096) == \
        pa.decode_workspace_bytes(d, 128, 4096, 0)
