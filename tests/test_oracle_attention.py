"""Pins of the oracle's attention and merge against what the pages fix.

* Algenta "Attention variant kernels": the score 8/sqrt(64) = 1.0, the stable
  softmax of [2, 1, 3], the online-softmax running state over values
  [10, 20, 30] ending at 24.20512484720024, the causal mask, GQA 32/8 = 4.
* NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache": end
  alignment, causal and windowed bands, rows with no key return zeros, the
  two-segment [6, 10] example with keys_before = 3.
* Library routine: torch's scaled_dot_product_attention (CPU, float64) with
  an explicit end-aligned causal mask.
* Invariants: constant V, one-hot V, future-key perturbation, GQA by head
  repetition, page placement, split-and-merge.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, brute, merge
from oracle.paged import PagedCache


def _dense_single(q, k, v, scale, window_left=-1):
    """q [n_q, D], k/v [n_kv, D] single head."""
    return attention.dense_attention(q[:, None, :], k[:, None, :], v[:, None, :], scale, window_left)


def test_p1_score_scaling_and_single_key(golden):
    g = golden("algenta_worked_values.json")["sdpa"]
    d = int(g["d"])
    q = np.zeros((1, d)); k = np.zeros((1, d))
    q[0, :8] = 1.0; k[0, :8] = 1.0                     # q.k = 8
    assert q[0] @ k[0] == g["qk"]
    v = np.arange(d, dtype=np.float64)[None, :] - 7.5
    out, lse = _dense_single(q, k, v, 1.0 / math.sqrt(d))
    assert lse[0, 0] == g["score"]                     # one key: lse = its score
    np.testing.assert_array_equal(out[0, 0], v[0])     # and returns V exactly


def _three_key_case(values):
    """q = e0, keys with q.k = [2, 1, 3] under scale 1."""
    d = max(4, np.asarray(values).shape[-1] if np.ndim(values) > 1 else 4)
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k = np.zeros((3, d)); k[:, 0] = [2.0, 1.0, 3.0]
    return q, k


def test_p2_stable_softmax_weights(golden):
    g = golden("algenta_worked_values.json")["stable_softmax"]
    q, k = _three_key_case(None)
    v = np.eye(3, 4)                                   # one-hot V reads out the weights
    out, lse = _dense_single(q, k, v, 1.0)
    w = out[0, 0, :3]
    assert abs(w[0] - g["weight_0"]) <= 1e-16
    assert abs(np.sum(w) - 1.0) <= 1e-15
    assert abs(lse[0, 0] - (g["row_max"] + math.log(g["sum_exp"]))) <= 1e-15


def test_p3_online_softmax_running_state(golden):
    g = golden("algenta_worked_values.json")["online_softmax"]
    trace, final = merge.online_softmax_trace(g["scores"], g["values"])
    for (m, l, o), m_ref, l_ref, o_ref in zip(trace, g["running_max"], g["running_sum"], g["running_out"]):
        assert m == m_ref
        assert abs(l - l_ref) <= 1e-15 * l_ref
        assert abs(o - o_ref) <= 1e-14 * o_ref
    assert abs(final - g["final"]) <= 1e-14
    # the plain oracle gives the same number
    q, k = _three_key_case(None)
    v = np.zeros((3, 4)); v[:, 0] = g["values"]
    out, _ = _dense_single(q, k, v, 1.0)
    assert abs(out[0, 0, 0] - g["final"]) <= 1e-13


def test_p4_lse_merge_of_chunks(golden):
    g = golden("algenta_worked_values.json")["online_softmax"]
    s, vals = g["scores"], g["values"]
    # chunk {0, 1}: max 2, l = 1 + e^-1, o = (10 + 20 e^-1) / l
    l01 = g["running_sum"][1]
    lse01 = 2.0 + math.log(l01)
    o01 = g["running_out"][1] / l01
    po = np.array([[[o01]], [[vals[2]]]])
    pl = np.array([[lse01], [s[2]]])
    out, lse = merge.lse_merge(po, pl, [0, 2])
    assert abs(out[0, 0, 0] - g["final"]) <= 1e-14
    assert abs(lse[0, 0] - (3.0 + math.log(g["running_sum"][2]))) <= 1e-15
    # one key per chunk reproduces the same result, in any chunk order
    po1 = np.array(vals, dtype=np.float64)[:, None, None]
    pl1 = np.array(s, dtype=np.float64)[:, None]
    for perm in ([0, 1, 2], [2, 0, 1], [1, 2, 0]):
        o, l = merge.lse_merge(po1[perm], pl1[perm], [0, 3])
        assert abs(o[0, 0, 0] - g["final"]) <= 1e-13
    # empty partials: zeros and -inf
    o, l = merge.lse_merge(np.ones((2, 1, 3)), np.full((2, 1), -np.inf), [0, 2])
    assert np.all(o == 0) and l[0, 0] == -np.inf
    # an empty chunk among live ones is ignored
    o, l = merge.lse_merge(np.array([[[5.0]], [[7.0]]]), np.array([[-np.inf], [0.5]]), [0, 2])
    assert o[0, 0, 0] == 7.0 and l[0, 0] == 0.5


def test_merge_matches_brute():
    rng = np.random.default_rng(5)
    po = rng.standard_normal((7, 2, 3))
    pl = rng.standard_normal((7, 2)) * 3
    pl[2, 1] = -np.inf
    offs = [0, 3, 3, 7]
    out, lse = merge.lse_merge(po, pl, offs)
    for r in range(3):
        for h in range(2):
            states = [(list(po[i, h]), float(pl[i, h])) for i in range(offs[r], offs[r + 1])]
            if not states:
                assert lse[r, h] == -np.inf and np.all(out[r, h] == 0)
                continue
            o, l = brute.merge_states(states)
            np.testing.assert_allclose(out[r, h], o, rtol=0, atol=1e-13)
            assert abs(lse[r, h] - l) <= 1e-13


def test_p5_constant_and_one_hot_values():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((9, 4, 16)); k = rng.standard_normal((12, 2, 16))
    out, _ = attention.dense_attention(q, k, np.ones((12, 2, 16)), 0.25)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-15)
    onehot = np.zeros((12, 2, 16)); onehot[np.arange(12), :, np.arange(12)] = 1.0
    out, _ = attention.dense_attention(q, k, onehot, 0.25)
    np.testing.assert_allclose(out[..., :12].sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(out[..., :12] >= 0)


def test_p6_causal_mask(golden):
    g = golden("algenta_worked_values.json")["causal_mask"]
    qpos, kpos = g["attend"]
    lo, hi = attention.visible_range(qpos, 8, 8, -1)
    assert lo <= kpos <= hi
    qpos, kpos = g["masked"]
    lo, hi = attention.visible_range(qpos, 8, 8, -1)
    assert not (lo <= kpos <= hi)
    # perturbing future keys/values leaves every row unchanged
    rng = np.random.default_rng(7)
    q = rng.standard_normal((8, 2, 8)); k = rng.standard_normal((8, 1, 8)); v = rng.standard_normal((8, 1, 8))
    out, lse = attention.dense_attention(q, k, v, 0.3)
    for t in range(8):
        k2, v2 = k.copy(), v.copy()
        k2[t + 1:] += 5.0; v2[t + 1:] -= 3.0
        o2, l2 = attention.dense_attention(q, k2, v2, 0.3)
        np.testing.assert_array_equal(o2[t], out[t])
        np.testing.assert_array_equal(l2[t], lse[t])


def test_p8_gqa_equals_repeated_heads(golden):
    g = golden("algenta_worked_values.json")["gqa"]
    assert g["n_query_heads"] // g["n_kv_heads"] == g["group"]
    rng = np.random.default_rng(8)
    hq, hkv = 8, 2
    q = rng.standard_normal((5, hq, 16)); k = rng.standard_normal((11, hkv, 16)); v = rng.standard_normal((11, hkv, 16))
    out, lse = attention.dense_attention(q, k, v, 0.25)
    kr = np.repeat(k, hq // hkv, axis=1); vr = np.repeat(v, hq // hkv, axis=1)
    o2, l2 = attention.dense_attention(q, kr, vr, 0.25)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)


@pytest.mark.parametrize("n_q,n_kv,window,after", [(7, 7, -1, 0), (3, 10, -1, 0), (1, 13, -1, 0), (6, 9, 2, 0),
                                                   (9, 9, 0, 0), (7, 7, -1, -1), (6, 9, 2, 3), (5, 12, -1, 4),
                                                   (9, 9, 0, 2), (3, 10, 1, -1)])
def test_p9_matches_torch_sdpa(n_q, n_kv, window, after):
    """The band of attention_packed (NumKong matrix-kernels page): row r of
    n_q queries over n_kv keys sees keys r + n_kv - n_q - keys_before through
    r + n_kv - n_q + keys_after, each side unbounded at None (-1 here)."""
    rng = np.random.default_rng(9)
    hq, hkv, d = 4, 2, 16
    q = rng.standard_normal((n_q, hq, d)); k = rng.standard_normal((n_kv, hkv, d)); v = rng.standard_normal((n_kv, hkv, d))
    scale = 0.37
    out, lse = attention.dense_attention(q, k, v, scale, window, after)
    i = np.arange(n_q)[:, None] + n_kv - n_q
    j = np.arange(n_kv)[None, :]
    mask = ((j <= i + after) if after >= 0 else True) & ((j >= i - window) if window >= 0 else True)
    mask = np.broadcast_to(mask, (n_q, n_kv)).copy()
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    s = scale * np.einsum("qhd,khd->hqk", q, np.repeat(k, hq // hkv, axis=1))
    ref_lse = torch.logsumexp(torch.from_numpy(np.where(mask[None], s, -np.inf)), dim=-1).numpy().T
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_q,n_kv,window,after,sinks", [(6, 30, 4, 0, 3), (1, 40, 9, 0, 4), (9, 9, 1, 2, 2)])
def test_p9b_sinks_match_torch_sdpa(n_q, n_kv, window, after, sinks):
    """Sink keys (Algenta streaming_llm_sink_score) as an explicit mask:
    key j is seen when j <= position + keys_after and (j >= position -
    keys_before or j < sinks)."""
    rng = np.random.default_rng(19)
    hq, hkv, d = 2, 1, 8
    q = rng.standard_normal((n_q, hq, d)); k = rng.standard_normal((n_kv, hkv, d)); v = rng.standard_normal((n_kv, hkv, d))
    out, lse = attention.dense_attention(q, k, v, 0.5, window, after, sinks)
    i = np.arange(n_q)[:, None] + n_kv - n_q
    j = np.arange(n_kv)[None, :]
    mask = (j <= i + after) & ((j >= i - window) | (j < sinks))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, hq, axis=1)).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(np.repeat(v, hq, axis=1)).permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.5).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


def test_p10_window_band(golden):
    g = golden("numkong_band_example.json")
    rng = np.random.default_rng(10)
    lens, offs = g["lengths"], g["offsets"]
    heads, depth, before = g["heads"], 16, g["keys_before"]
    T = offs[-1]
    q = rng.standard_normal((T, heads, depth)); k = rng.standard_normal((T, heads, depth)); v = rng.standard_normal((T, heads, depth))
    scale = 1 / 4
    # the band: each row sees itself and the 3 keys before it -> at most 4 keys
    for L in lens:
        for r in range(L):
            lo, hi = attention.visible_range(r, L, L, before)
            assert hi == r and lo == max(0, r - before) and hi - lo + 1 <= g["window_keys"]
    cache, pt = _pack_contiguous(k, v, offs, 16)
    out, lse = attention.ragged_paged_attention(q, offs, lens, cache, pt, scale, before)
    bo, bl = brute.ragged_attention(q.tolist(), offs, lens,
                                    [k[offs[s]:offs[s + 1]].tolist() for s in range(2)],
                                    [v[offs[s]:offs[s + 1]].tolist() for s in range(2)], scale, before)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-13)
    # a window at least as long as the keys changes nothing
    o_full, l_full = attention.ragged_paged_attention(q, offs, lens, cache, pt, scale, -1)
    o_w, l_w = attention.ragged_paged_attention(q, offs, lens, cache, pt, scale, max(lens) - 1)
    np.testing.assert_array_equal(o_full, o_w)
    np.testing.assert_array_equal(l_full, l_w)


def test_p10b_band_after_the_row(golden):
    """keys_after > 0 (attention_packed's band): brute force on the
    two-segment example, the band's edges, and the special cases -- a
    single-token row is its segment's last position, so keys after it do not
    exist; a keys_after that reaches every segment's end is unbounded."""
    g = golden("numkong_band_example.json")
    rng = np.random.default_rng(12)
    lens, offs = g["lengths"], g["offsets"]
    T = offs[-1]
    q = rng.standard_normal((T, 2, 8)); k = rng.standard_normal((T, 2, 8)); v = rng.standard_normal((T, 2, 8))
    cache, pt = _pack_contiguous(k, v, offs, 16)
    ks = [k[offs[s]:offs[s + 1]].tolist() for s in range(2)]
    vs = [v[offs[s]:offs[s + 1]].tolist() for s in range(2)]
    for before, after in ((3, 2), (-1, 1), (0, -1), (-1, -1), (2, 5)):
        for L in lens:
            for r in range(L):
                lo, hi = attention.visible_range(r, L, L, before, after)
                assert hi == (L - 1 if after < 0 else min(r + after, L - 1))
                assert lo == (0 if before < 0 else max(0, r - before))
        out, lse = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, before, window_right=after)
        bo, bl = brute.ragged_attention(q.tolist(), offs, lens, ks, vs, 0.3, before, after)
        np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-13)
    o_u, l_u = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, -1, window_right=-1)
    o_m, l_m = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, -1, window_right=max(lens) - 1)
    np.testing.assert_array_equal(o_u, o_m)
    np.testing.assert_array_equal(l_u, l_m)
    # unbounded on both sides: every row is the plain softmax over all its segment's keys
    for s in range(2):
        a, b = offs[s], offs[s + 1]
        sc = 0.3 * np.einsum("qhd,khd->hqk", q[a:b], k[a:b])
        w = np.exp(sc - sc.max(-1, keepdims=True))
        ref = np.einsum("hqk,khd->qhd", w / w.sum(-1, keepdims=True), v[a:b])
        np.testing.assert_allclose(o_u[a:b], ref, rtol=0, atol=1e-13)
    # one query row over 9 keys: keys after its position do not exist
    q1 = rng.standard_normal((1, 2, 8)); k9 = rng.standard_normal((9, 2, 8)); v9 = rng.standard_normal((9, 2, 8))
    o0, l0 = attention.dense_attention(q1, k9, v9, 0.5, 4, 0)
    for after in (1, 7, -1):
        o1, l1 = attention.dense_attention(q1, k9, v9, 0.5, 4, after)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)


def test_p10c_streaming_sinks(golden):
    """Algenta streaming_llm_sink_score: 4 sink tokens plus a 20-token
    window over 100 positions attend positions 0-3 and 80-99 from the last
    position; here window_left = window - 1 and sink_keys = n_sink.  Also:
    brute force, sinks 0 = the band, sinks reaching the band = one range."""
    g = golden("algenta_streaming_sink.json")
    n = g["seq_len"]
    idx = attention.visible_keys(0, 1, n, g["window_size"] - 1, 0, g["n_sink_tokens"])   # one row, at position n - 1
    seen = np.zeros(n); seen[idx] = 1.0
    assert [seen[p] for p in g["positions"]] == g["scores"]
    assert list(idx) == list(range(4)) + list(range(80, 100))
    # the attention over that set is the plain softmax over exactly those keys
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 1, 8)); k = rng.standard_normal((n, 1, 8)); v = rng.standard_normal((n, 1, 8))
    out, lse = attention.dense_attention(q, k, v, 0.4, g["window_size"] - 1, 0, g["n_sink_tokens"])
    sc = 0.4 * (k[idx, 0] @ q[0, 0])
    w = np.exp(sc - sc.max())
    np.testing.assert_allclose(out[0, 0], (w / w.sum()) @ v[idx, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], sc.max() + np.log(w.sum()), rtol=0, atol=1e-14)
    # brute force on the two-segment example, several bands with sinks
    gb = golden("numkong_band_example.json")
    lens, offs = gb["lengths"], gb["offsets"]
    T = offs[-1]
    q = rng.standard_normal((T, 2, 8)); k = rng.standard_normal((T, 2, 8)); v = rng.standard_normal((T, 2, 8))
    cache, pt = _pack_contiguous(k, v, offs, 16)
    ks = [k[offs[s]:offs[s + 1]].tolist() for s in range(2)]
    vs = [v[offs[s]:offs[s + 1]].tolist() for s in range(2)]
    for before, after, sinks in ((2, 0, 2), (1, 1, 3), (0, 0, 1), (3, -1, 2), (-1, 0, 4)):
        out, lse = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, before, window_right=after,
                                                    sink_keys=sinks)
        bo, bl = brute.ragged_attention(q.tolist(), offs, lens, ks, vs, 0.3, before, after, sinks)
        np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-13)
    o_b, l_b = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, 2)
    o_0, l_0 = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, 2, sink_keys=0)
    np.testing.assert_array_equal(o_b, o_0)
    # sinks covering every key before any band: the causal rows from key 0
    # (sinks widen the band's left side only; keys after a row stay hidden)
    o_c, l_c = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, -1)
    o_s, l_s = attention.ragged_paged_attention(q, offs, lens, cache, pt, 0.3, 1, sink_keys=max(lens))
    np.testing.assert_array_equal(o_c, o_s)
    np.testing.assert_array_equal(l_c, l_s)


def test_rows_with_no_key_are_zero():
    rng = np.random.default_rng(11)
    # 5 query rows over 3 keys: rows 0 and 1 sit at positions -2, -1
    q = rng.standard_normal((5, 2, 8)); k = rng.standard_normal((3, 1, 8)); v = rng.standard_normal((3, 1, 8))
    out, lse = attention.dense_attention(q, k, v, 0.5)
    assert np.all(out[:2] == 0) and np.all(lse[:2] == -np.inf)
    assert np.all(np.isfinite(lse[2:]))
    # a zero-length KV segment
    out, lse = attention.dense_attention(q[:1], k[:0], v[:0], 0.5)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def _pack_contiguous(k, v, offs, page_size, perm_seed=None):
    """Pack per-segment K/V rows into a float64 f32-typed paged cache."""
    B = len(offs) - 1
    hkv, d = k.shape[1], k.shape[2]
    counts = [-(-(offs[s + 1] - offs[s]) // page_size) for s in range(B)]
    total = sum(counts)
    ids = np.arange(total) if perm_seed is None else np.random.default_rng(perm_seed).permutation(total)
    pt = np.zeros((B, max(counts)), dtype=np.int64)
    at = 0
    for s in range(B):
        pt[s, :counts[s]] = ids[at:at + counts[s]]
        at += counts[s]
    cache = PagedCache("f32", total, hkv, page_size, d)
    for s in range(B):
        for j in range(offs[s + 1] - offs[s]):
            for h in range(hkv):
                cache.store(pt, s, j, h, k[offs[s] + j, h], v[offs[s] + j, h])
    return cache, pt


def test_page_placement_invariance():
    rng = np.random.default_rng(12)
    offs = [0, 20, 53, 54]
    lens = [20, 33, 1]
    k = rng.standard_normal((54, 2, 8)); v = rng.standard_normal((54, 2, 8))
    q = rng.standard_normal((54, 4, 8))
    c1, p1 = _pack_contiguous(k, v, offs, 4)
    c2, p2 = _pack_contiguous(k, v, offs, 4, perm_seed=3)
    o1, l1 = attention.ragged_paged_attention(q, offs, lens, c1, p1, 0.3, -1)
    o2, l2 = attention.ragged_paged_attention(q, offs, lens, c2, p2, 0.3, -1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_split_kv_then_merge_equals_full():
    rng = np.random.default_rng(13)
    L, d = 1000, 16
    q = rng.standard_normal((1, 4, d)); k = rng.standard_normal((L, 2, d)); v = rng.standard_normal((L, 2, d))
    full_o, full_l = attention.dense_attention(q, k, v, 0.25)
    for split in (1, 64, 333, 512, 1000):
        chunks = [(a, min(a + split, L)) for a in range(0, L, split)]
        po, pl = [], []
        for a, b in chunks:
            # the decode row sees every key; a chunk is the same row over keys a..b-1
            o, l = attention.dense_attention(q, k[a:b], v[a:b], 0.25)
            po.append(o[0]); pl.append(l[0])
        out, lse = merge.lse_merge(np.array(po), np.array(pl), [0, len(chunks)])
        np.testing.assert_allclose(out[0], full_o[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0], full_l[0], rtol=0, atol=1e-12)
