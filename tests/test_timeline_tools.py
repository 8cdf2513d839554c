"""The placement helpers of paged_kv_cache_158_amd/timeline.py (no GPU):
CU numbers from the hardware-id fields, and the average number of other
waves that shared a wave's SIMD or CU while it ran."""
import importlib.util
import os

import numpy as np

_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "paged_kv_cache_158_amd", "timeline.py")


def _timeline():
    spec = importlib.util.spec_from_file_location("pa_timeline_tools", _PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_import_leaves_the_library_choice_alone():
    before = os.environ.get("PA_LIBRARY")
    mod = _timeline()
    assert os.environ.get("PA_LIBRARY") == before
    assert mod.pa is None and mod.torch is None


def test_cu_ids_take_the_cu_sh_se_and_xcc_fields():
    t = _timeline()
    # HW_ID: CU in bits 8..11, SH in bit 12, SE in bits 13..15; SIMD (bits
    # 4..5) and wave slot (bits 0..3) do not change the CU
    hw = np.array([(3 << 8) | (1 << 12) | (2 << 13) | (2 << 4) | 5,
                   (3 << 8) | (1 << 12) | (2 << 13),
                   (4 << 8) | (1 << 12) | (2 << 13),
                   (3 << 8) | (1 << 12) | (2 << 13)], dtype=np.int64)
    xcc = np.array([0, 0, 0, 6])
    cu = t._cu_ids(xcc, hw)
    assert cu[0] == cu[1]
    assert len({int(cu[1]), int(cu[2]), int(cu[3])}) == 3
    # every field combination maps to its own number
    fields = [(x, se, sh, c) for x in range(8) for se in range(8) for sh in range(2) for c in range(16)]
    hw = np.array([(c << 8) | (sh << 12) | (se << 13) for _, se, sh, c in fields], dtype=np.int64)
    ids = t._cu_ids(np.array([f[0] for f in fields]), hw)
    assert len(set(ids.tolist())) == len(fields)


def test_peers_is_the_time_averaged_count_of_other_waves():
    t = _timeline()
    key = np.array([1, 1, 2, 1, 1])
    st = np.array([0., 5, 0, 20, 0])
    en = np.array([10., 15, 10, 30, 10])
    p = t._peers(key, st, en, st, en)
    # wave 0 [0, 10): wave 1 for 5 of 10, wave 4 for all 10 -> 1.5;
    # wave 1 [5, 15): waves 0 and 4 for 5 of 10 each -> 1.0
    assert np.allclose(p, [1.5, 1.0, 0.0, 0.0, 1.5])
    # the others counted over another interval (e.g. whole lives) than the
    # wave's own (e.g. its streaming)
    p2 = t._peers(key, np.array([5., 5, 0, 20, 5]), en, st, en)
    assert np.allclose(p2, [2.0, 1.0, 0.0, 0.0, 2.0])
