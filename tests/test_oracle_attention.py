"""Pins for the oracle cache write, gather and attention.

The oracle's paged result is checked against things other than itself:
torch's scaled_dot_product_attention (float64, CPU) on each request's K/V
taken straight from the script (never through the pool), closed forms,
invariance under relabelling of physical blocks, and chunking invariance
of causal prefill.  A test at the end plants plausible mistakes in the
oracle and checks that these pins catch them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import synth
from oracle import attention, run
from oracle.attention import to_f64


def logical_kv(w):
    """Per sequence id, its token K/V rows in order, from the script alone."""
    toks = {}
    for step in list(w.history) + [w.final]:
        i = 0
        for op in step.ops:
            if op[0] == "new":
                toks[op[1]] = []
            elif op[0] == "fork":
                toks[op[2]] = list(toks[op[1]])
            elif op[0] == "append":
                for _ in range(op[2]):
                    toks[op[1]].append((step.k[i], step.v[i]))
                    i += 1
            elif op[0] == "prompt":
                # every prompt row, whether or not a prefix cache would skip it
                toks[op[1]] = [(step.k[i + j], step.v[i + j]) for j in range(len(op[2]))]
                i += len(op[2])
            elif op[0] == "free":
                del toks[op[1]]
    out = {}
    for sid, rows in toks.items():
        if rows:
            k = np.stack([to_f64(r[0], w.dtype) for r in rows])
            v = np.stack([to_f64(r[1], w.dtype) for r in rows])
            if getattr(w, "kv_dtype", None) == "fp8":
                k, v = torch_fp8_round_trip(k, w.k_scale), torch_fp8_round_trip(v, w.v_scale)
        else:
            k = v = np.zeros((0, w.num_kv_heads, w.head_dim))
        out[sid] = (k, v)
    return out


def torch_fp8_round_trip(x, scale):
    """x [L][Hkv][D] stored in E4M3 with per-head scales and read back, by
    torch's float8_e4m3fn conversion (saturating at 448 first; torch would
    give NaN beyond it): independent of the oracle's codec."""
    sc = torch.from_numpy(np.asarray(scale, np.float32))[None, :, None]
    y = (torch.from_numpy(x.astype(np.float32)) / sc).clamp(-448.0, 448.0)
    back = y.to(torch.float8_e4m3fn).to(torch.float64) * sc.double()
    return back.numpy()


def sdpa(qrows, K, V, scale, causal):
    """torch SDPA on one sequence: q [Lq][H][D], K/V [L][Hkv][D] → [Lq][H][D]."""
    q = torch.from_numpy(qrows).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(q, k, v, scale=scale, is_causal=causal, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def library_reference(w, seed=5):
    """Output of the final step computed by torch from contiguous K/V."""
    kv = logical_kv(w)
    qf = to_f64(w.q, w.dtype)
    out = np.zeros(qf.shape)
    if w.kind == "decode":
        for r, sid in enumerate(w.batch):
            K, V = kv[int(sid)]
            if K.shape[0]:
                out[r] = sdpa(qf[r:r + 1], K, V, w.scale, False)[0]
        return out
    # varlen: a causal chunk of q_len rows at the end of an L-token sequence is
    # the last q_len rows of full causal self-attention; the earlier rows get
    # arbitrary queries and are discarded.
    rng = np.random.default_rng(seed)
    qlen = {}
    for op in w.final.ops:
        if op[0] == "append":
            qlen[op[1]] = qlen.get(op[1], 0) + op[2]
    row = 0
    for sid in w.batch:
        sid = int(sid)
        n = qlen.get(sid, 0)
        if n == 0:
            continue
        K, V = kv[sid]
        L = K.shape[0]
        full_q = rng.standard_normal((L, w.num_heads, w.head_dim))
        full_q[L - n:] = qf[row:row + n]
        out[row:row + n] = sdpa(full_q, K, V, w.scale, True)[L - n:]
        row += n
    return out


ALL = list(synth.FULL)


@pytest.mark.parametrize("name", ALL)
def test_paged_equals_contiguous_library_attention(name):
    w = synth.reduced(name)
    st = run.run_script(w)
    got = run.attend(w, st)
    ref = library_reference(w)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_context_len_reading_without_the_new_token():
    # reading where the step attends before its own token is written: the
    # same answer as the library over the first ctx-1 tokens
    w = synth.tiny_f32()
    st = run.run_script(w)
    lens = st.context_lens - 1
    got = attention.decode(w.q, st.k_cache, st.v_cache, st.block_tables, lens, w.scale,
                           w.dtype, w.num_kv_heads)
    kv = logical_kv(w)
    qf = to_f64(w.q, w.dtype)
    for r, sid in enumerate(w.batch):
        K, V = kv[int(sid)]
        ref = sdpa(qf[r:r + 1], K[:-1], V[:-1], w.scale, False)[0]
        np.testing.assert_allclose(got[r], ref, rtol=0, atol=1e-12)


def test_cache_write_is_exact_and_touches_only_its_slots():
    w = synth.reduced("gqa_decode_b32")
    st = run.run_script(w)
    kc0, vc0 = st.k_cache.copy(), st.v_cache.copy()
    slots = st.step_slots[-1]
    n = len(slots)
    rng = np.random.default_rng(3)
    k = rng.integers(0, 2**16, size=(n, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    v = rng.integers(0, 2**16, size=(n, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    sm = slots.copy()
    sm[1] = -1  # a skipped token
    attention.cache_write(k, v, sm, st.k_cache, st.v_cache)
    flat_k = st.k_cache.reshape(-1, w.num_kv_heads, w.head_dim)
    flat_k0 = kc0.reshape(-1, w.num_kv_heads, w.head_dim)
    for i, s in enumerate(sm):
        if s >= 0:
            assert (flat_k[s] == k[i]).all()
    untouched = np.ones(flat_k.shape[0], bool)
    untouched[sm[sm >= 0]] = False
    assert (flat_k[untouched] == flat_k0[untouched]).all()
    assert (flat_k[slots[1]] == flat_k0[slots[1]]).all()


def test_bf16_decoding_of_stored_bits():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80, 0x0001], np.uint16)
    vals = to_f64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625 and math.copysign(1, vals[4]) < 0 and np.isinf(vals[5])
    assert vals[6] == 2.0 ** -133  # smallest bf16 subnormal


def _one_seq_cache(K, V, B=4, perm_seed=0):
    """Place contiguous K/V [L][Hkv][D] into a pool through a permuted table."""
    L, hkv, d = K.shape
    nblk = -(-L // B)
    pool = nblk + 3
    table = np.random.default_rng(perm_seed).permutation(pool)[:nblk]
    kc = np.full((pool, B, hkv, d), np.nan)
    vc = np.full((pool, B, hkv, d), np.nan)
    for t in range(L):
        kc[table[t // B], t % B] = K[t]
        vc[table[t // B], t % B] = V[t]
    return kc, vc, table


def _dec(q, K, V, scale, B=4, perm_seed=0):
    kc, vc, table = _one_seq_cache(K, V, B, perm_seed)
    return attention.decode(q[None], kc.astype(np.float32), vc.astype(np.float32),
                            table[None], [K.shape[0]], scale, "f32", K.shape[1])[0]


def test_closed_forms():
    rng = np.random.default_rng(11)
    hkv, G, d = 2, 2, 8
    q = rng.standard_normal((hkv * G, d)).astype(np.float32)
    # one token: the output is that token's V row, whatever the score
    K = rng.standard_normal((1, hkv, d)).astype(np.float32)
    V = rng.standard_normal((1, hkv, d)).astype(np.float32)
    out = _dec(q, K, V, 0.3)
    for h in range(hkv * G):
        assert (out[h] == V[0, h // G].astype(np.float64)).all()
    # all V rows equal: output equals that row for every head
    L = 9
    K = rng.standard_normal((L, hkv, d)).astype(np.float32)
    V = np.repeat(rng.standard_normal((1, hkv, d)).astype(np.float32), L, 0)
    out = _dec(q, K, V, 0.3)
    for h in range(hkv * G):
        np.testing.assert_allclose(out[h], V[0, h // G], rtol=0, atol=1e-12)
    # zero query: uniform weights, the mean of the V rows
    V = rng.standard_normal((L, hkv, d)).astype(np.float32)
    out = _dec(np.zeros_like(q), K, V, 0.3)
    for h in range(hkv * G):
        np.testing.assert_allclose(out[h], V[:, h // G].astype(np.float64).mean(0), atol=1e-12)
    # two tokens: out = v1 + logistic(z0 - z1) (v0 - v1)
    K2, V2 = K[:2].astype(np.float64), V[:2].astype(np.float64)
    out = _dec(q, K[:2], V[:2], 0.3)
    for h in range(hkv * G):
        g = h // G
        z = 0.3 * (K2[:, g] @ q[h].astype(np.float64))
        np.testing.assert_allclose(out[h], V2[1, g] + expit(z[0] - z[1]) * (V2[0, g] - V2[1, g]),
                                   rtol=0, atol=1e-12)


def test_empty_context_gives_zeros():
    w = synth.decode_workload("edge", [0, 5, 0], num_heads=4, num_kv_heads=2, head_dim=8,
                              block_size=4, num_blocks=8, dtype="f32", seed=2)
    st = run.run_script(w)
    out = run.attend(w, st)
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.abs(out[1]).sum() > 0


def test_physical_relabelling_invariance():
    w = synth.reduced("parallel_sampling_cow")
    base = run.attend(w, run.run_script(w))
    for seed in (1, 2):
        w.free_order = np.random.default_rng(seed).permutation(w.num_blocks).astype(np.int32)
        st = run.run_script(w)
        got = run.attend(w, st)
        assert (got == base).all()  # the gather order depends only on logical position


def _swap_round_trip(w, st, move):
    """Swap the blocks of sequences 0 and 2 out to a CPU pool, clobber them on
    the GPU pool, swap them back in to other free blocks, and relabel the
    tables (SourceAIX page §6.2.1 steps (3)-(4)).  Returns (pool K, pool V,
    tables) after the round trip; `move` does the block moves."""
    kc, vc = st.k_cache.copy(), st.v_cache.copy()
    tabs = st.block_tables.copy()
    B = w.block_size
    used = sorted({int(b) for s in (0, 2) for b in tabs[s][: -(-int(st.context_lens[s]) // B)]})
    taken = {int(b) for b in tabs.ravel() if b >= 0}
    free = [b for b in range(w.num_blocks) if b not in taken][: len(used)]
    assert len(free) == len(used)
    host_k = np.zeros((len(used),) + kc.shape[1:], kc.dtype)
    host_v = np.zeros_like(host_k)
    move(kc, vc, host_k, host_v, [(b, i) for i, b in enumerate(used)])  # swap out
    kc[used] = 0x7FC1 if w.dtype == "bf16" else np.nan  # the GPU blocks are reused
    vc[used] = kc[used]
    move(host_k, host_v, kc, vc, [(i, f) for i, f in enumerate(free)])  # swap in
    relabel = dict(zip(used, free))
    for s in (0, 2):
        tabs[s] = [relabel.get(int(b), int(b)) for b in tabs[s]]
    return kc, vc, tabs


def test_swap_out_and_in_leaves_attention_unchanged():
    w = synth.reduced("gqa_decode_b32")
    st = run.run_script(w)
    base = attention.decode(w.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                            w.scale, w.dtype, w.num_kv_heads)
    kc, vc, tabs = _swap_round_trip(w, st, attention.swap_blocks)
    got = attention.decode(w.q, kc, vc, tabs, st.context_lens, w.scale, w.dtype, w.num_kv_heads)
    assert (got == base).all()
    assert not (tabs == st.block_tables).all()
    # a move that drops V, or moves the wrong block, changes the output
    def only_k(sk, sv, dk, dv, moves):
        for a, b in moves:
            dk[b] = sk[a]
    kc2, vc2, tabs2 = _swap_round_trip(w, st, only_k)
    bad = attention.decode(w.q, kc2, vc2, tabs2, st.context_lens, w.scale, w.dtype,
                           w.num_kv_heads)
    assert not np.isfinite(bad[0]).all() or not (bad[0] == base[0]).all()
    def shifted(sk, sv, dk, dv, moves):
        attention.swap_blocks(sk, sv, dk, dv, [(a, moves[(i + 1) % len(moves)][1])
                                                for i, (a, _) in enumerate(moves)])
    kc3, vc3, tabs3 = _swap_round_trip(w, st, shifted)
    bad3 = attention.decode(w.q, kc3, vc3, tabs3, st.context_lens, w.scale, w.dtype,
                            w.num_kv_heads)
    assert not (bad3[0] == base[0]).all()
    assert (bad3[1] == base[1]).all()  # sequence 1 kept its blocks


def test_chunked_prefill_equals_one_chunk_and_decode_rows_equal_decode():
    # one 30-token causal chunk after 20 prior tokens, and the same 30 rows
    # split into chunks of 12 and 18 over 20 and 32 prior tokens
    w = synth.varlen_workload("c", [(20, 30), (7, 1)], num_heads=4, num_kv_heads=2,
                              head_dim=16, block_size=4, num_blocks=64, dtype="bf16", seed=9)
    st = run.run_script(w)
    one = run.attend(w, st)
    qsl = np.array([0, 12, 30], np.int32)
    lens = np.array([32, 50], np.int32)
    tabs = np.stack([st.block_tables[0], st.block_tables[0]])
    split = attention.varlen(w.q[:30], qsl, lens, st.k_cache, st.v_cache, tabs, w.scale,
                             w.dtype, w.num_kv_heads)
    np.testing.assert_allclose(split, one[:30], rtol=0, atol=1e-12)
    dec = attention.decode(w.q[30:31], st.k_cache, st.v_cache, st.block_tables[1:2],
                           st.context_lens[1:2], w.scale, w.dtype, w.num_kv_heads)
    np.testing.assert_allclose(dec[0], one[30], rtol=0, atol=1e-12)


def test_sampled_outputs_match_full():
    w = synth.reduced("mixed_varlen")
    st = run.run_script(w)
    full = run.attend(w, st)
    rows = [(0, 0), (5, 7), (len(w.q) - 1, 31)]
    part = run.attend(w, st, rows)
    for r, h in rows:
        assert (part[r, h] == full[r, h]).all()
    w2 = synth.reduced("gqa_decode_b32")
    st2 = run.run_script(w2)
    full2 = run.attend(w2, st2)
    part2 = run.attend(w2, st2, [(1, 3), (5, 31)])
    assert (part2[1, 3] == full2[1, 3]).all() and (part2[5, 31] == full2[5, 31]).all()


# --- the pins catch plausible mistakes ---------------------------------------

def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(attention, name, fn)


@pytest.mark.parametrize("mistake", ["swapped_index", "head_mod", "no_scale", "causal_off_by_one"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "swapped_index":
        def bad(table, length, B):
            return [int(table[t % B]) * B + t // B if t % B < len(table) else 0
                    for t in range(length)]
        _planted(monkeypatch, "logical_rows", bad)
        w = synth.reduced("gqa_decode_b32")
    elif mistake == "head_mod":
        orig = attention.decode

        def bad(q, kc, vc, bt, cl, scale, dtype, hkv, pairs=None):
            # query head h read KV head h % hkv instead of h // G
            n, H, D = q.shape
            G = H // hkv
            perm = [(h % hkv) * G + (h // hkv) for h in range(H)]
            return orig(q[:, perm], kc, vc, bt, cl, scale, dtype, hkv, pairs)[:, np.argsort(perm)]
        monkeypatch.setattr(run.attention, "decode", bad)
        w = synth.reduced("gqa_decode_b32")
    elif mistake == "no_scale":
        orig = attention._attend
        _planted(monkeypatch, "_attend", lambda q, K, V, s: orig(q, K, V, 1.0))
        w = synth.reduced("gqa_decode_b32")
    else:
        orig = attention._attend
        _planted(monkeypatch, "_attend", lambda q, K, V, s: orig(q, K[:-1], V[:-1], s)
                 if K.shape[0] > 1 else orig(q, K, V, s))
        w = synth.reduced("mixed_varlen")
    st = run.run_script(w)
    got = run.attend(w, st)
    ref = library_reference(w)
    assert not np.allclose(got, ref, rtol=0, atol=1e-6)
