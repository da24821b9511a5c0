"""The seeded generators: shapes, ranges, page tables, reproducibility, and
the work accounting (pinned to the Algenta page's KV-cache byte example)."""

import math

import numpy as np
import pytest

import synth
from synth import work


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_shapes_and_pages(k):
    w = synth.make(k)
    assert w.num_q_heads % w.num_kv_heads == 0
    assert np.all(w.q_lens <= w.kv_lens) and np.all(w.q_lens >= 1)
    used = []
    for s in range(w.num_seqs):
        n = -(-int(w.kv_lens[s]) // w.page_size)
        used.extend(w.page_table[s, :n].tolist())
    assert sorted(used) == list(range(w.num_pages))       # every page once
    assert w.q_offsets[-1] == w.total_q
    if k == 2:
        assert w.kv_lens.min() >= 512 and w.kv_lens.max() <= 4096 and w.num_seqs == 32
    if k == 3:
        assert w.total_q == 8192 and list(w.q_lens) == [128, 256, 512, 768, 1024, 1536, 1792, 2176]
    if k == 4:
        assert np.all((w.q_lens[:4] >= 1024) & (w.q_lens[:4] <= 4096))
        assert np.all((w.kv_lens[4:] >= 2048) & (w.kv_lens[4:] <= 8192)) and w.window_left == 1023
    if k == 5:
        assert w.kv_lens.min() >= 4096 and w.kv_lens.max() <= 32768 and w.num_seqs == 128


def test_reproducible_and_subset_identical():
    w = synth.make(2)
    a, b = synth.new_tokens(w), synth.new_tokens(w)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
    sub = w.subset([3, 17])
    ta = synth.new_tokens(sub)
    np.testing.assert_array_equal(ta["q"], a["q"][[3, 17]])
    K1, V1, _, _ = synth.prior_rows(w, 17)
    K2, V2, _, _ = synth.prior_rows(sub, 1)
    np.testing.assert_array_equal(K1, K2)
    np.testing.assert_array_equal(V1, V2)


def test_fp8_prior_rows_are_oracle_quantised():
    from oracle import formats
    w = synth.make(5).subset([0])
    K, V, ks, vs = synth.prior_rows(w, 0)
    rng = np.random.default_rng([w.seed, 2, 0])
    Kf = rng.standard_normal(K.shape, dtype=np.float32).astype(np.float64)
    codes, scale = formats.fp8_quantize(Kf[:200])
    np.testing.assert_array_equal(scale, ks[:200].astype(np.float64))
    # the library cast and the oracle's encoder agree on all but rare double-rounding ties
    assert np.mean(codes == K[:200]) > 0.999


def test_qk_norm_unit_rms():
    w = synth.make(4).subset([0, 10])
    nt = synth.new_tokens(w)
    from oracle import formats
    q = formats.bf16_value(nt["q"])
    rms = np.sqrt(np.mean(q * q, axis=-1))
    assert np.all(np.abs(rms - 1) < 1e-2)


def test_kv_bytes_formula_pin(golden):
    g = golden("algenta_worked_values.json")["kv_cache_bytes"]
    assert work.kv_cache_memory_bytes(g["layers"], g["heads"], g["d_head"], g["seq_len"], g["batch"]) == g["bytes"]
    # the decode byte count's K+V term is the same footprint per layer
    w = synth.make(2).subset([0])
    w.kv_lens[:] = 4096
    w.num_kv_heads, w.head_dim = 32, 128
    kv_term = work.decode_bytes(w) - (w.num_q_heads * w.head_dim * 4 + 256 * 4 + w.num_q_heads * 4)
    assert kv_term * g["layers"] == g["bytes"]


def test_work_numbers():
    assert work.prefill_pairs(synth.make(3)) == sum(L * (L + 1) // 2 for L in synth.make(3).q_lens)
    w4 = synth.make(4)
    pairs = sum(sum(min(i + 1, 1024) for i in range(L)) for L in w4.q_lens[:4])
    assert work.prefill_pairs(w4) == pairs
    assert abs(work.prefill_flops(synth.make(3)) / 1e9 - 100.73) < 0.01
