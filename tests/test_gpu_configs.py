"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times, against the oracle (the oracle regenerates exactly the
compared sequences' inputs from their own random streams).

For each workload: RoPE + append then attention run over the whole batch on
the GPU; for the compared sequences the oracle computes q_out, the appended
cache rows and out/lse.  Compared: every sequence of the tiny, batched-decode
and prefill workloads; every prefill segment of the mixed workload plus 16 of
its decode rows (the shortest, the longest and 14 drawn); 16 sequences of the
long-context e4m3 workload (its 4 longest, its shortest and 11 drawn).
Checked: stored q_out and appended K/V rows (e4m3 codes and scales included)
bit-equal to the oracle's; every other cache byte unchanged; out and lse
within the workload's tolerance, with the margin recorded for the run's
summary.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import formats
from oracle.paged import k_storage_to_logical, v_storage_to_logical
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SAMPLES = {
    1: None,                     # everything
    2: None,
    3: None,
    4: "mixed",
    5: "long",
}


def _sample(w, how):
    if how is None:
        return np.arange(w.num_seqs)
    rng = np.random.default_rng(99)
    if how == "mixed":
        pre = np.nonzero(w.q_lens > 1)[0]
        dec = np.nonzero(w.q_lens == 1)[0]
        dec_sorted = dec[np.argsort(w.kv_lens[dec], kind="stable")]
        ends = dec_sorted[[0, -1]]
        mid = rng.choice(dec_sorted[1:-1], size=14, replace=False)
        return np.unique(np.concatenate([pre, ends, mid]))
    order = np.argsort(w.kv_lens, kind="stable")
    fixed = np.concatenate([order[:1], order[-4:]])
    mid = rng.choice(order[1:-4], size=11, replace=False)
    return np.unique(np.concatenate([fixed, mid]))


def _written_mask(w):
    m = np.zeros((w.num_pages, w.num_kv_heads, w.page_size), bool)
    for s in range(w.num_seqs):
        L, ql = int(w.kv_lens[s]), int(w.q_lens[s])
        for j in range(L - ql, L):
            m[int(w.page_table[s][j // w.page_size]), :, j % w.page_size] = True
    return m


def _cache_rows(w, k_pages, v_pages, seq, slots, page_table):
    """Rows [n, heads, D] of K (blocks of 32 NK dims) and V (16-byte runs in
    MFMA operand order), raw storage elements."""
    pages = page_table[seq][slots // w.page_size].astype(np.int64)
    offs = slots % w.page_size
    k = k_storage_to_logical(w.cache_dtype, k_pages[pages])   # [n, heads, P, D]
    v = v_storage_to_logical(w.cache_dtype, v_pages[pages])   # [n, heads, D, P]
    n = np.arange(len(slots))
    return k[n, :, offs, :], v[n, :, :, offs]


def _raw(t, dtype):
    """CPU tensor -> numpy raw storage (float32 / uint16 bf16 bits / uint8 codes)."""
    if dtype == "f32":
        return t.numpy()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def _values(raw, dtype):
    if dtype == "f32":
        return raw.astype(np.float64)
    if dtype == "bf16":
        return formats.bf16_value(raw)
    return formats.e4m3_value(raw)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_full_size(k):
    w = synth.make(k)
    gu.say(f"workload {k} {w.name}: B={w.num_seqs} T={w.total_q} max_kv={w.max_kv_len}")
    d = gu.to_device(w)
    q_out, out, lse = gu.run_hip(w, d)
    torch.cuda.synchronize()
    gu.say(f"workload {k}: GPU done")

    seqs = _sample(w, SAMPLES[k])
    ws = w.subset(seqs)
    raw_sub = synth.build_cache(ws)
    q_o, cache_o, out_o, lse_o = gu.oracle_run(ws, raw_sub)
    tok = ws.token_ids

    # --- q_out
    qg = gu.host_values(q_out, w.in_dtype)[tok]
    frac = gu.compare_storage(qg, q_o, w.in_dtype, "q_out")
    gu.say(f"workload {k}: q_out differing fraction {frac:.2e}")

    # --- appended cache rows of the sampled sequences
    c = d["cache"]
    kg_all = c.k_pages.cpu()
    vg_all = c.v_pages.cpu()
    kg_raw, vg_raw = _raw(kg_all, w.cache_dtype), _raw(vg_all, w.cache_dtype)
    ok_adj = 0
    for i, s in enumerate(seqs):
        L, ql = int(w.kv_lens[s]), int(w.q_lens[s])
        slots = np.arange(L - ql, L)
        kr_, vr_ = _cache_rows(w, kg_raw, vg_raw, s, slots, w.page_table)
        kg, vg = _values(kr_, w.cache_dtype), _values(vr_, w.cache_dtype)
        ko = cache_o.k[ws.page_table[i][slots // w.page_size].astype(np.int64), :, slots % w.page_size, :]
        vo = cache_o.v[ws.page_table[i][slots // w.page_size].astype(np.int64), :, :, slots % w.page_size]
        if w.cache_dtype == "e4m3":
            kcg, vcg = kr_, vr_
            kco, vco = formats.e4m3_code(ko), formats.e4m3_code(vo)
            for a, b, what in ((kcg, kco, "K codes"), (vcg, vco, "V codes")):
                ok_adj += int(np.sum(a != b))
                assert np.array_equal(a, b), f"{what}: {int(np.sum(a != b))} codes differ from the oracle's"
            pages = w.page_table[s][slots // w.page_size]
            opages = ws.page_table[i][slots // w.page_size]
            for sc_g, sc_o in ((c.k_scales.cpu().numpy(), cache_o.k_scale), (c.v_scales.cpu().numpy(), cache_o.v_scale)):
                g_ = sc_g[pages, :, slots % w.page_size].astype(np.float64)
                o_ = sc_o[opages, :, slots % w.page_size]
                assert np.array_equal(g_, o_), "scales differ from the oracle's"
        else:
            gu.compare_storage(kg, ko, w.cache_dtype, "K rows")
            gu.compare_storage(vg, vo, w.cache_dtype, "V rows")
    gu.say(f"workload {k}: appended rows bit-exact")

    # --- nothing else in the cache changed
    raw = d["raw_cache"]
    mask = _written_mask(w)
    nb = kg_all.shape[2]
    kb = kg_all.view(torch.uint8).numpy().reshape(w.num_pages, w.num_kv_heads, nb, w.page_size, -1)
    kr = raw["k_pages"].view(np.uint8).reshape(kb.shape)
    kb, kr = np.transpose(kb, (0, 1, 3, 2, 4)), np.transpose(kr, (0, 1, 3, 2, 4))   # slot before block
    assert np.array_equal(kb[~mask], kr[~mask]), "K bytes outside the appended slots changed"
    # V: compare element bit patterns in logical [page][head][dim][slot] order
    vb = v_storage_to_logical(w.cache_dtype, vg_raw)
    vr = v_storage_to_logical(w.cache_dtype, raw["v_pages"].reshape(vg_raw.shape))
    if w.cache_dtype == "f32":
        vb, vr = vb.view(np.uint32), vr.view(np.uint32)
    assert np.all((vb == vr) | mask[:, :, None, :]), "V bytes outside the appended slots changed"
    gu.say(f"workload {k}: untouched bytes ok")

    # --- attention output
    tol = gu.tol_for(w)
    og = gu.host_values(out, w.in_dtype)[tok]
    lg = lse.cpu().numpy().astype(np.float64)[tok]
    e_out = gu.check_close(og, out_o, tol, "out")
    e_lse = gu.check_close(lg, lse_o, tol, "lse")
    gu.record_margin(f"workload {k} {w.name} ({len(seqs)}/{w.num_seqs} seqs)", e_out, e_lse, tol)
    gu.say(f"workload {k}: out max err {e_out:.3g}, lse max err {e_lse:.3g} (tol {tol})")
