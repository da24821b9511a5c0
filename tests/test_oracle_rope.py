"""Pins of the oracle's RoPE + append, and a brute-force cross-check of the
whole oracle (RoPE + append + attention) on shrunken versions of the five
workloads.

What the pages fix: rotary embedding preserves norms, is the identity at
position 0, and makes q.k depend only on the position difference; the
interleaved layout pairs adjacent components and the half layout pairs the
two halves (Mojo page, ``interleaved`` parameter; aria_kernel ``rope`` /
``rope_half``); partial rotary leaves the dims past ``rotary_dim`` alone
(aria_kernel ``rope_half_partial``); p-RoPE pairs (i, i + D/2) and rotates
only the first pairs, with the full head_dim denominator (aria_kernel
``rope_half_proportional``); M-RoPE splits the pairs into sections, each
rotated by its own position stream (Mojo ``mrope_section``); the RoPE angle
of pair i at position p is p * base**(-2i/d) (Algenta, "Five ways to inject
position").
"""

import math

import numpy as np
import pytest

import synth
from synth.configs import Workload, _pages
from oracle import attention, brute, formats, rope
from oracle.paged import PagedCache


def _table(max_pos, rotary_dim, base):
    half = rotary_dim // 2
    t = np.zeros((max_pos, half, 2))
    for p in range(max_pos):
        for i in range(half):
            a = p * base ** (-2.0 * i / rotary_dim)
            t[p, i] = (math.cos(a), math.sin(a))
    return t


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_identity_at_position_zero(layout):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 4, 64))
    t = _table(1, 64, 1e4)
    y = rope.rotate(x, t[0, :, 0], t[0, :, 1], 64, layout)
    np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_norm_preserved_and_relative_position(layout):
    rng = np.random.default_rng(1)
    d, R = 32, 32
    t = _table(200, R, 100.0)
    q = rng.standard_normal(d); k = rng.standard_normal(d)
    for p in (0, 1, 17, 150):
        y = rope.rotate(q, t[p, :, 0], t[p, :, 1], R, layout)
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
    def dot(m, n):
        return rope.rotate(q, t[m, :, 0], t[m, :, 1], R, layout) @ rope.rotate(k, t[n, :, 0], t[n, :, 1], R, layout)
    for m, n in ((3, 10), (40, 47), (100, 107)):
        assert abs(dot(m, n) - dot(m - 3, n - 3)) < 1e-12
    assert abs(dot(5, 5) - q @ k) < 1e-12


def test_rotation_direction_and_pairing():
    # pair 0 has angle p (base**0 = 1): (1, 0) -> (cos p, sin p)
    t = _table(4, 8, 1e4)
    x = np.zeros(8); x[0] = 1.0
    y = rope.rotate(x, t[3, :, 0], t[3, :, 1], 8, "half")
    assert y[0] == math.cos(3) and y[4] == math.sin(3)
    y = rope.rotate(x, t[3, :, 0], t[3, :, 1], 8, "interleaved")
    assert y[0] == math.cos(3) and y[1] == math.sin(3)
    # interleaved applied to a vector equals half applied to its pair-gathered copy
    rng = np.random.default_rng(2)
    z = rng.standard_normal(8)
    perm = np.array([0, 2, 4, 6, 1, 3, 5, 7])          # half position -> interleaved position
    yi = rope.rotate(z, t[2, :, 0], t[2, :, 1], 8, "interleaved")
    yh = rope.rotate(z[perm], t[2, :, 0], t[2, :, 1], 8, "half")
    np.testing.assert_array_equal(yi[perm], yh)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_partial_rotary_leaves_tail(layout):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 256))
    t = _table(9, 128, 1e4)
    y = rope.rotate(x, t[8, :, 0], t[8, :, 1], 128, layout)
    np.testing.assert_array_equal(y[:, 128:], x[:, 128:])
    assert not np.allclose(y[:, :128], x[:, :128])


def test_proportional_layout():
    """aria_kernel rope_half_proportional (p-RoPE): the rotate-half pairing
    over the whole head, (i, i + D/2); only the first pairs rotate, the rest
    stay identity; with every pair rotated it is plain rope_half; frequencies
    use the full head_dim denominator."""
    rng = np.random.default_rng(4)
    D, R = 64, 32                                    # 16 of 32 pairs rotate
    t = _table(50, D, 1e4)[:, :R // 2]               # full-head denominator, first R/2 pairs
    x = rng.standard_normal((3, D))
    y = rope.rotate(x, t[7, :, 0], t[7, :, 1], R, "half_proportional")
    rot = np.r_[0:R // 2, D // 2:D // 2 + R // 2]
    keep = np.setdiff1d(np.arange(D), rot)
    np.testing.assert_array_equal(y[:, keep], x[:, keep])              # the other pairs are identity
    assert not np.allclose(y[:, rot], x[:, rot])
    # pairing: dim 0 goes with dim D/2 (not R/2 as in the partial layout)
    e0 = np.zeros(D); e0[0] = 1.0
    z = rope.rotate(e0, t[3, :, 0], t[3, :, 1], R, "half_proportional")
    assert z[0] == math.cos(3) and z[D // 2] == math.sin(3) and z[R // 2] == 0.0
    # every pair rotated: the plain rotate-half layout
    tf = _table(50, D, 1e4)
    np.testing.assert_array_equal(rope.rotate(x, tf[9, :, 0], tf[9, :, 1], D, "half_proportional"),
                                  rope.rotate(x, tf[9, :, 0], tf[9, :, 1], D, "half"))
    # identity at 0, norms kept, q.k a function of the position difference
    np.testing.assert_array_equal(rope.rotate(x, t[0, :, 0], t[0, :, 1], R, "half_proportional"), x)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    assert abs(np.linalg.norm(rope.rotate(q, t[40, :, 0], t[40, :, 1], R, "half_proportional")) -
               np.linalg.norm(q)) < 1e-12
    def dot(m, n):
        return (rope.rotate(q, t[m, :, 0], t[m, :, 1], R, "half_proportional") @
                rope.rotate(k, t[n, :, 0], t[n, :, 1], R, "half_proportional"))
    assert abs(dot(12, 19) - dot(2, 9)) < 1e-12
    # brute force agrees
    for p in (0, 5, 31):
        b = brute.rope_row(list(x[1]), list(t[p, :, 0]), list(t[p, :, 1]), R, "half_proportional")
        np.testing.assert_allclose(rope.rotate(x[1], t[p, :, 0], t[p, :, 1], R, "half_proportional"),
                                   np.array(b), rtol=0, atol=1e-15)
    # the synthetic table of a proportional workload uses the full head_dim denominator
    w = synth.custom(q_lens=[3], kv_lens=[3], num_q_heads=2, num_kv_heads=1, head_dim=D, rotary_dim=R,
                     rope_layout="half_proportional", rope_theta=1e4)
    np.testing.assert_array_equal(synth.freqs_table(w), _table(w.max_pos, D, 1e4)[:, :R // 2].astype(np.float32))


def _mrope_run(q, k, sections, pos_streams, t, layout="half"):
    """Rotate [T, 1, D] rows through the oracle's fused step with M-RoPE."""
    T, _, D = q.shape
    R = 2 * sum(sections)
    from oracle.paged import PagedCache as PC
    cache = PC("f32", 1, 1, 16, D)
    q_out, c2 = rope.rope_qk_write_paged(q, k, k, "f32", [0, T], [T], np.asarray(pos_streams), t, R, layout,
                                         cache, np.array([[0]]), mrope_sections=sections)
    kk = np.array([c2.k[0, 0, j] for j in range(T)])
    return q_out, kk


def test_mrope_sections():
    """Mojo mrope_section: the head dimension split across modalities; each
    section of pairs rotates by its own position stream.  One section, or
    every stream equal, is plain RoPE; a stream moves only its own pairs;
    q.k depends only on the per-section position differences."""
    rng = np.random.default_rng(5)
    D, T = 64, 6
    sections = [8, 16, 8]                                   # pairs: 32 = R/2 with R = D
    t = _table(100, D, 1e4)
    q = rng.standard_normal((T, 1, D)); k = rng.standard_normal((T, 1, D))
    base = np.array([3, 9, 14, 20, 27, 41])
    same = np.stack([base, base, base])
    for layout in ("half", "interleaved"):
        q_m, k_m = _mrope_run(q, k, sections, same, t, layout)
        q_p = formats.storage_round(rope.rotate(q, t[base, :, 0][:, None, :], t[base, :, 1][:, None, :], D, layout), "f32")
        np.testing.assert_array_equal(q_m, q_p)
        q_1, _ = _mrope_run(q, k, [32], base[None, :], t, layout)
        np.testing.assert_array_equal(q_1, q_p)
        # a different stream for section 1 moves only section 1's pairs (and their partners)
        streams = np.stack([base, base + 7, base])
        q_d, _ = _mrope_run(q, k, sections, streams, t, layout)
        a_idx, b_idx = rope.pair_indices(D, layout, D)
        sec = np.repeat(np.arange(3), sections)
        moved = np.zeros(D, dtype=bool)
        moved[a_idx[sec == 1]] = True
        moved[b_idx[sec == 1]] = True
        np.testing.assert_array_equal(q_d[:, :, ~moved], q_m[:, :, ~moved])
        assert not np.allclose(q_d[:, :, moved], q_m[:, :, moved])
    # pair positions follow the sections in pair order
    pp = rope.pair_positions(np.stack([base, base + 1, base + 2]), sections, D)
    assert pp.shape == (T, 32) and (pp[:, :8] == base[:, None]).all() and (pp[:, 8:24] == base[:, None] + 1).all()
    # relative position per section: shifting every stream by the same amount keeps q.k
    def dots(streams):
        qm, km = _mrope_run(q, k, sections, streams, t)
        return qm[0, 0] @ km[5]
    s1 = np.stack([base, base + 2, base + 5])
    assert abs(dots(s1) - dots(s1 + 4)) < 1e-4                # float32 storage rounding
    assert abs(dots(s1) - dots(np.stack([base, 2 * base, base + 5]))) > 1e-3    # section 1's differences change
    with pytest.raises(ValueError):
        rope.pair_positions(same, [8, 8, 8], D)               # must count R/2 pairs


def test_slots_follow_the_append():
    # segment lengths: q 2 over kv 7 -> slots 5, 6; q 3 over kv 3 -> 0, 1, 2
    seq, slot, pos = rope.token_slots([0, 2, 5], [7, 3])
    assert list(seq) == [0, 0, 1, 1, 1] and list(slot) == [5, 6, 0, 1, 2]
    assert list(pos) == list(slot)
    _, _, pos = rope.token_slots([0, 2, 5], [7, 3], [9, 9, 4, 5, 6])
    assert list(pos) == [9, 9, 4, 5, 6]


def test_synth_table_is_the_rope_angle():
    w = synth.make(1)
    t = synth.freqs_table(w)
    ref = _table(w.max_pos, w.rotary_dim, w.rope_theta)
    np.testing.assert_array_equal(t, ref.astype(np.float32))


# ----------------------------------------------------------------- brute force
def _tiny(k):
    """Shrunken workload k: same dtypes, layouts, GQA ratio, window kind and
    page size as workload k, a few tokens."""
    mk = lambda **a: Workload(**a)  # noqa: E731
    rng = np.random.default_rng(100 + k)
    if k == 1:
        q_lens, kv_lens = np.array([5, 12]), np.array([5, 12])
        kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, rotary_dim=64, rope_layout="half",
                  rope_theta=1e4, page_size=16, in_dtype="f32", cache_dtype="f32",
                  softmax_scale=1 / 8, window_left=-1, qk_norm=False, explicit_positions=True)
        order = "identity"
    elif k == 2:
        q_lens, kv_lens = np.array([1, 1, 1]), np.array([17, 3, 40])
        kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=32, rotary_dim=32, rope_layout="half",
                  rope_theta=5e5, page_size=16, in_dtype="bf16", cache_dtype="bf16",
                  softmax_scale=0.25, window_left=-1, qk_norm=False, explicit_positions=False)
        order = "permuted"
    elif k == 3:
        q_lens, kv_lens = np.array([3, 20, 9]), np.array([3, 20, 9])
        kw = dict(num_q_heads=4, num_kv_heads=1, head_dim=32, rotary_dim=32, rope_layout="half",
                  rope_theta=5e5, page_size=16, in_dtype="bf16", cache_dtype="bf16",
                  softmax_scale=0.25, window_left=-1, qk_norm=False, explicit_positions=True)
        order = "in_order"
    elif k == 4:
        q_lens, kv_lens = np.array([12, 1, 1]), np.array([12, 40, 7])
        kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=32, rotary_dim=16, rope_layout="interleaved",
                  rope_theta=1e4, page_size=32, in_dtype="bf16", cache_dtype="bf16",
                  softmax_scale=1.0, window_left=4, qk_norm=True, explicit_positions=True)
        order = "permuted"
    else:
        q_lens, kv_lens = np.array([1, 1]), np.array([33, 18])
        kw = dict(num_q_heads=8, num_kv_heads=1, head_dim=64, rotary_dim=64, rope_layout="half",
                  rope_theta=1e6, page_size=16, in_dtype="bf16", cache_dtype="e4m3",
                  softmax_scale=0.25, window_left=-1, qk_norm=False, explicit_positions=False)
        order = "permuted"
    table, npages = _pages(rng, kv_lens, kw["page_size"], order)
    w = mk(name=f"tiny{k}", seed=100 + k, q_lens=q_lens.astype(np.int32), kv_lens=kv_lens.astype(np.int32),
           page_table=table, num_pages=npages, split_tokens=0, **kw)
    w.seq_ids = np.arange(w.num_seqs); w.token_ids = np.arange(w.total_q); w.full_total_q = w.total_q
    return w


def _k_raw(k_pages, w, page, head, d, t):
    """Element (dim d, slot t) of a K page-head block, by the header's offset
    formula on the flattened block."""
    nk = 2 if w.cache_dtype == "e4m3" else 1
    idx = ((d // (32 * nk)) * w.page_size + t) * 32 * nk + ((d % 32) // 8) * nk * 8 + ((d // 32) % nk) * 8 + d % 8
    return k_pages[page, head].reshape(-1)[idx]


def _v_raw(v_pages, w, page, head, d, t):
    """Element (dim d, slot t) of a V page-head block, by the header's offset
    formula on the flattened block."""
    nv = {"f32": 1, "bf16": 2, "e4m3": 4}[w.cache_dtype]
    D = w.head_dim
    c = (d // 16) // nv
    idx = ((t // 16) * (D // (16 * nv)) + c) * 64 * 4 * nv + (16 * ((t % 16) // 4) + d % 16) * 4 * nv \
        + ((d // 16) % nv) * 4 + t % 4
    return v_pages[page, head].reshape(-1)[idx]


def _values(dtype, raw):
    if dtype == "f32":
        return raw.astype(np.float64)
    if dtype == "bf16":
        return formats.bf16_value(raw)
    return formats.e4m3_value(raw)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_brute_force_matches_oracle(k):
    w = _tiny(k)
    nt = synth.new_tokens(w)
    q, kk, v = (_values(w.in_dtype, nt[n]) for n in ("q", "k", "v"))
    table = synth.freqs_table(w).astype(np.float64)
    raw = synth.build_cache(w, threads=1)
    cache = PagedCache.from_storage(w.cache_dtype, raw["k_pages"], raw["v_pages"], raw["k_scales"], raw["v_scales"])
    q_out, cache2 = rope.rope_qk_write_paged(q, kk, v, w.in_dtype, w.q_offsets, w.kv_lens, w.position_ids,
                                             table, w.rotary_dim, w.rope_layout, cache, w.page_table)
    out, lse = attention.ragged_paged_attention(q_out, w.q_offsets, w.kv_lens, cache2, w.page_table,
                                                w.softmax_scale, w.window_left)

    # brute force: rotate each row in pure Python, place rows by hand, attend
    pos = w.positions
    offs = w.q_offsets
    bq = []
    for t in range(w.total_q):
        c, s = table[pos[t], :, 0].tolist(), table[pos[t], :, 1].tolist()
        bq.append([formats.storage_round(np.array(brute.rope_row(q[t, h].tolist(), c, s, w.rotary_dim, w.rope_layout)),
                                         w.in_dtype).tolist() for h in range(w.num_q_heads)])
    np.testing.assert_array_equal(np.array(bq), q_out)
    keys, vals = [], []
    for s in range(w.num_seqs):
        L, ql = int(w.kv_lens[s]), int(w.q_lens[s])
        ks, vs = [], []
        for j in range(L):
            page, off = int(w.page_table[s][j // w.page_size]), j % w.page_size
            krow, vrow = [], []
            for h in range(w.num_kv_heads):
                if j >= L - ql:                                  # appended now
                    t = offs[s] + j - (L - ql)
                    c, sn = table[pos[t], :, 0].tolist(), table[pos[t], :, 1].tolist()
                    kr = brute.rope_row(kk[t, h].tolist(), c, sn, w.rotary_dim, w.rope_layout)
                    if w.cache_dtype == "e4m3":
                        kc, ksc = formats.fp8_quantize(np.array(kr))
                        vc, vsc = formats.fp8_quantize(v[t, h])
                        kr = (formats.e4m3_value(kc) * ksc).tolist()
                        vr = (formats.e4m3_value(vc) * vsc).tolist()
                    else:
                        kr = formats.storage_round(np.array(kr), w.cache_dtype).tolist()
                        vr = formats.storage_round(v[t, h], w.cache_dtype).tolist()
                else:                                            # prior rows, read raw
                    kr = _values(w.cache_dtype, np.array([_k_raw(raw["k_pages"], w, page, h, dd, off)
                                                          for dd in range(w.head_dim)]))
                    vr = _values(w.cache_dtype, np.array([_v_raw(raw["v_pages"], w, page, h, dd, off)
                                                          for dd in range(w.head_dim)]))
                    if w.cache_dtype == "e4m3":
                        kr = kr * float(raw["k_scales"][page, h, off])
                        vr = vr * float(raw["v_scales"][page, h, off])
                    kr, vr = kr.tolist(), vr.tolist()
                krow.append(kr); vrow.append(vr)
            ks.append(krow); vs.append(vrow)
        keys.append(ks); vals.append(vs)
    bo, bl = brute.ragged_attention(np.array(bq).tolist(), list(offs), list(w.kv_lens), keys, vals,
                                    w.softmax_scale, w.window_left)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)
    # every slot the step wrote is now finite, and nothing else changed
    written = np.zeros((w.num_pages, w.num_kv_heads, w.page_size), bool)
    for s in range(w.num_seqs):
        for j in range(int(w.kv_lens[s]) - int(w.q_lens[s]), int(w.kv_lens[s])):
            written[int(w.page_table[s][j // w.page_size]), :, j % w.page_size] = True
    before_k = np.transpose(cache.k, (0, 1, 2, 3))
    same = ~written
    np.testing.assert_array_equal(np.isnan(cache2.k[same]), np.isnan(before_k[same]))
    assert np.all(np.isfinite(cache2.k[written]))
