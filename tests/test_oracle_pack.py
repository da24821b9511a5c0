"""Pins of the oracle's pack (NumKong matrix-kernels page, "Attention with a
Pre-Packed KV-Cache" and attention_pack): what it stores is read back
through the cache's own addressing and compared with the input rows; page
assignment, kept lengths and e4m3 rows against their definitions; attention
over the pack against the pure-Python brute force on the row slices."""

import numpy as np
import pytest

from oracle import attention as o_attn
from oracle import brute, formats
from oracle import pack as o_pack


def _rows(rng, n, hkv, d, dtype):
    x = rng.standard_normal((n, hkv, d))
    return formats.bf16_round(x) if dtype in ("bf16", "e4m3") else formats.f32_round(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_round_trip_is_the_row_slices(dtype):
    rng = np.random.default_rng(1)
    offs = [0, 5, 5, 40, 41, 77]                  # an empty slot, a one-key slot
    lens = [3, 0, 35, 1, 20]                     # fewer keys than the slot in two segments
    k, v = _rows(rng, 80, 2, 64, dtype), _rows(rng, 80, 2, 64, dtype)
    cache, table, kept = o_pack.attention_pack(k, v, offs, lens, dtype, 16)
    assert list(kept) == lens
    for s in range(5):
        K, V = cache.gather(table, s, int(kept[s]))
        assert np.array_equal(K, k[offs[s]:offs[s] + lens[s]])
        assert np.array_equal(V, v[offs[s]:offs[s] + lens[s]])


def test_pages_in_segment_order_and_disjoint():
    kept = np.array([17, 0, 16, 1, 33])
    first, counts = o_pack.page_assignment(kept, 16)
    assert list(counts) == [2, 0, 1, 1, 3]
    assert list(first) == [0, 2, 2, 3, 4]
    rng = np.random.default_rng(2)
    offs = np.concatenate([[0], np.cumsum(kept + 3)])    # slots 3 keys longer than kept
    k = _rows(rng, int(offs[-1]), 1, 64, "bf16")
    cache, table, _ = o_pack.attention_pack(k, k, offs, kept, "bf16", 16)
    used = [int(table[s, i]) for s in range(5) for i in range(counts[s])]
    assert used == list(range(7)) and cache.num_pages == 7


def test_kept_length_clamps():
    offs = [0, 10, 30]
    assert list(o_pack.kept_lengths(offs)) == [10, 20]                  # whole slots by default
    assert list(o_pack.kept_lengths(offs, [12, -3])) == [10, 0]         # never past the slot, never negative
    assert list(o_pack.kept_lengths(offs, None, 15)) == [10, 15]        # the stated maximum


def test_e4m3_rows():
    rng = np.random.default_rng(3)
    k = _rows(rng, 20, 2, 64, "e4m3") * 7.0
    k[4, 1] = 0.0                                              # an all-zero row: scale 0, zero codes
    cache, table, kept = o_pack.attention_pack(k, k, [0, 20], None, "e4m3", 16)
    pg = table[0][np.arange(20) // 16]
    sl = np.arange(20) % 16
    for j in range(20):
        for h in range(2):
            amax = np.max(np.abs(k[j, h]))
            sc = cache.k_scale[pg[j], h, sl[j]]
            assert sc == np.float32(amax / 448.0)
            codes = cache.k[pg[j], h, sl[j]]
            if amax == 0:
                assert sc == 0 and np.all(codes == 0)
                continue
            assert np.max(np.abs(codes)) == 448.0 or np.isclose(np.max(np.abs(codes)) * sc, amax, rtol=2 ** -4)
            # e4m3 keeps 3 mantissa bits: half a step relative, or half the
            # smallest subnormal step (2^-9) absolute
            err = np.abs(codes * sc - k[j, h])
            assert np.all(err <= np.maximum(np.abs(k[j, h]) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 1e-12))


@pytest.mark.parametrize("window", [(-1, 0), (4, 0), (3, 2)])
def test_attention_over_pack_is_brute_force_on_slices(window):
    rng = np.random.default_rng(4)
    offs = [0, 9, 9, 30, 31]
    lens = [7, 0, 21, 1]
    q_lens = [3, 0, 6, 1]
    hq, hkv, d = 4, 2, 64
    k, v = _rows(rng, 31, hkv, d, "bf16"), _rows(rng, 31, hkv, d, "bf16")
    q = _rows(rng, sum(q_lens), hq, d, "bf16")
    q_offsets = np.concatenate([[0], np.cumsum(q_lens)])
    cache, table, kept = o_pack.attention_pack(k, v, offs, lens, "bf16", 16)
    out, lse = o_attn.ragged_paged_attention(q, q_offsets, kept, cache, table, 0.125, window[0],
                                             window_right=window[1])
    keys = [[[list(k[offs[s] + j, g]) for g in range(hkv)] for j in range(lens[s])] for s in range(4)]
    vals = [[[list(v[offs[s] + j, g]) for g in range(hkv)] for j in range(lens[s])] for s in range(4)]
    qq = [[list(q[t, h]) for h in range(hq)] for t in range(q.shape[0])]
    bo, bl = brute.ragged_attention(qq, list(q_offsets), lens, keys, vals, 0.125, window[0], window[1])
    assert np.allclose(out, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12, equal_nan=False)
