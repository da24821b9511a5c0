"""GPU parity of nk_attention_pack (NumKong matrix-kernels page, "Attention
with a Pre-Packed KV-Cache" and attention_pack): ragged K/V token rows with
cumulative key_offsets and optional key_lengths are packed into the paged
cache, then attended over with kv_lens = the kept lengths.  The pack is
integer and byte work: kept lengths, page-table rows and every stored
element (e4m3 codes and scales included) are compared bit for bit with the
oracle's pack; attention over the pack to the usual tolerances."""

import zlib

import numpy as np
import pytest
import torch

from oracle import attention as o_attn
from oracle import formats
from oracle import pack as o_pack
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (slots, kept lengths or None, q_lens, hq, hkv, D, P, cache dtype)
CASES = {
    "bf16_d128_p16_gaps": ([70, 0, 203, 1, 50, 300], [65, 0, 200, 1, 50, 299], [65, 0, 37, 1, 1, 1], 8, 2, 128, 16,
                           "bf16"),
    "bf16_d64_p32_whole_slots": ([33, 64, 5, 97], None, [33, 1, 5, 20], 4, 4, 64, 32, "bf16"),
    "e4m3_d128_p16": ([70, 203, 1, 300], [60, 203, 1, 250], [60, 40, 1, 1], 8, 2, 128, 16, "e4m3"),
    "bf16_d256_p32": ([90, 17, 120], [80, 17, 119], [80, 1, 30], 4, 2, 256, 32, "bf16"),
    "f32_d64_p16": ([9, 45, 130], [9, 40, 128], [9, 12, 1], 4, 2, 64, 16, "f32"),
}


def _inputs(name, slots, lens, hkv, d, dtype, rng):
    offs = np.concatenate([[0], np.cumsum(slots)]).astype(np.int32)
    rows = int(offs[-1])
    k = rng.standard_normal((rows, hkv, d))
    v = rng.standard_normal((rows, hkv, d))
    if dtype == "f32":
        k, v = formats.f32_round(k), formats.f32_round(v)
        dk = torch.from_numpy(k.astype(np.float32)).cuda()
        dv = torch.from_numpy(v.astype(np.float32)).cuda()
    else:
        kb, vb = formats.bf16_bits(formats.bf16_round(k)), formats.bf16_bits(formats.bf16_round(v))
        k, v = formats.bf16_value(kb), formats.bf16_value(vb)
        dk = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
        dv = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    return offs, k, v, dk, dv


def _host_cache(cache, dtype):
    conv = (lambda t: t.cpu().numpy()) if dtype != "bf16" else (lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16))
    ks = None if cache.k_scales is None else cache.k_scales.cpu().numpy()
    vs = None if cache.v_scales is None else cache.v_scales.cpu().numpy()
    return PagedCache.from_storage(dtype, conv(cache.k_pages), conv(cache.v_pages), ks, vs)


@pytest.mark.parametrize("name", sorted(CASES))
def test_pack_parity(name):
    slots, lens, q_lens, hq, hkv, d, P, cdt = CASES[name]
    gu.say(f"pack {name}: slots={slots} kept={lens} q_lens={q_lens} D={d} P={P} cache={cdt}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    offs, k, v, dk, dv = _inputs(name, slots, lens, hkv, d, cdt, rng)
    d_offs = torch.from_numpy(offs).cuda()
    d_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32).cuda()
    cache, kv_lens, max_len = nk.attention_pack(dk, dv, d_offs, d_lens, page_size=P, cache_dtype=cdt)
    torch.cuda.synchronize()

    o_cache, o_table, kept = o_pack.attention_pack(k, v, offs, lens, cdt, P)
    assert np.array_equal(kv_lens.cpu().numpy(), kept)
    table = cache.page_table.cpu().numpy()
    first, counts = o_pack.page_assignment(kept, P)
    for s in range(len(kept)):
        assert np.array_equal(table[s, :counts[s]], o_table[s, :counts[s]])
    g_cache = _host_cache(cache, cdt)
    for s in range(len(kept)):
        n = int(kept[s])
        if n == 0:
            continue
        pg = o_table[s][np.arange(n) // P]
        sl = np.arange(n) % P
        assert np.array_equal(g_cache.k[pg, :, sl, :], o_cache.k[pg, :, sl, :]), f"K of segment {s}"
        assert np.array_equal(g_cache.v[pg, :, :, sl], o_cache.v[pg, :, :, sl]), f"V of segment {s}"
        if cdt == "e4m3":
            assert np.array_equal(g_cache.k_scale[pg, :, sl], o_cache.k_scale[pg, :, sl])
            assert np.array_equal(g_cache.v_scale[pg, :, sl], o_cache.v_scale[pg, :, sl])

    # attention over the pack: queries aligned to the end of each segment's kept keys
    q_offsets = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(q_offsets[-1])
    qv = rng.standard_normal((T, hq, d))
    if cdt == "f32":
        qv = formats.f32_round(qv)
        dq = torch.from_numpy(qv.astype(np.float32)).cuda()
    else:
        qb = formats.bf16_bits(formats.bf16_round(qv))
        qv = formats.bf16_value(qb)
        dq = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    scale = 1.0 / np.sqrt(d)
    lse = torch.empty(T, hq, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(dq, torch.from_numpy(q_offsets).cuda(), kv_lens, cache, scale,
                                         max(q_lens), max_len, -1, lse=lse)
    torch.cuda.synchronize()
    out_o, lse_o = o_attn.ragged_paged_attention(qv, q_offsets, kept, o_cache, o_table, scale, -1)
    tol = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}[cdt]
    og = out.cpu().numpy().astype(np.float64) if cdt == "f32" else gu.host_values(out, "bf16")
    gu.check_close(og, out_o, tol, "out")
    gu.check_close(lse.cpu().numpy(), lse_o, tol, "lse")


def test_pack_attention_backward_rows():
    """Pack with spare room, attention under a window with sink keys, then
    the gradients with dk/dv at the pack's input rows: rows of kept keys
    match the oracle; the spare rows past each kept length are untouched."""
    slots, kept_in, q_lens, hq, hkv, d, P = [70, 203, 1, 300], [65, 200, 1, 250], [65, 37, 1, 1], 8, 2, 128, 16
    wl, sinks = 40, 4
    gu.say("pack + attention + backward rows")
    rng = np.random.default_rng(2024)
    offs, k, v, dk_in, dv_in = _inputs("bwd", slots, kept_in, hkv, d, "bf16", rng)
    d_offs = torch.from_numpy(offs).cuda()
    cache, kv_lens, max_len = nk.attention_pack(dk_in, dv_in, d_offs, torch.tensor(kept_in, dtype=torch.int32).cuda(),
                                                page_size=P)
    q_offsets = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(q_offsets[-1])
    qb = formats.bf16_bits(formats.bf16_round(rng.standard_normal((T, hq, d))))
    gb = formats.bf16_bits(formats.bf16_round(rng.standard_normal((T, hq, d))))
    dq_t = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    dout = torch.from_numpy(gb.view(np.int16)).cuda().view(torch.bfloat16)
    scale = 1.0 / np.sqrt(d)
    d_qoffs = torch.from_numpy(q_offsets).cuda()
    lse = torch.empty(T, hq, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(dq_t, d_qoffs, kv_lens, cache, scale, max(q_lens), max_len, wl, lse=lse,
                                         sink_keys=sinks)
    rows = int(offs[-1])
    dk = torch.full((rows, hkv, d), 7.0, dtype=torch.float32, device="cuda")
    dv = torch.full((rows, hkv, d), 7.0, dtype=torch.float32, device="cuda")
    dq, dk, dv = nk.ragged_paged_attention_backward(dq_t, d_qoffs, kv_lens, cache, scale, max_len, out, dout, lse,
                                                    d_offs, rows, wl, 0, sinks, dk=dk, dv=dv)
    torch.cuda.synchronize()

    o_cache, o_table, kept = o_pack.attention_pack(k, v, offs, kept_in, "bf16", P)
    dq_o, dk_o, dv_o = o_attn.ragged_paged_attention_backward(formats.bf16_value(qb), q_offsets, kept, o_cache,
                                                              o_table, scale, formats.bf16_value(gb), wl, 0, sinks)
    dqg, dkg, dvg = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    sc = max(1.0, float(np.max(np.abs(dq_o))))
    gu.check_close(dqg / sc, dq_o / sc, 2e-2, "dq")
    for s in range(len(slots)):
        a, n = int(offs[s]), int(kept[s])
        sk = max(1.0, float(np.max(np.abs(dk_o[s])))) if n else 1.0
        sv = max(1.0, float(np.max(np.abs(dv_o[s])))) if n else 1.0
        gu.check_close(dkg[a:a + n] / sk, dk_o[s] / sk, 2e-2, f"dk segment {s}")
        gu.check_close(dvg[a:a + n] / sv, dv_o[s] / sv, 2e-2, f"dv segment {s}")
        assert np.all(dkg[a + n:int(offs[s + 1])] == 7.0) and np.all(dvg[a + n:int(offs[s + 1])] == 7.0)


def test_pack_backward_default_gradient_buffers():
    """Gradients into the binding's own dk/dv buffers, over a pack with spare
    room: rows of kept keys match the oracle, rows past each kept length (keys
    no row reads) are zeros."""
    slots, kept_in, q_lens, hq, hkv, d, P = [40, 90, 17], [33, 90, 5], [33, 20, 1], 4, 2, 64, 16
    gu.say("pack + backward into default buffers")
    rng = np.random.default_rng(2025)
    offs, k, v, dk_in, dv_in = _inputs("bwd_default", slots, kept_in, hkv, d, "bf16", rng)
    d_offs = torch.from_numpy(offs).cuda()
    cache, kv_lens, max_len = nk.attention_pack(dk_in, dv_in, d_offs, torch.tensor(kept_in, dtype=torch.int32).cuda(),
                                                page_size=P)
    q_offsets = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(q_offsets[-1])
    qb = formats.bf16_bits(formats.bf16_round(rng.standard_normal((T, hq, d))))
    gb = formats.bf16_bits(formats.bf16_round(rng.standard_normal((T, hq, d))))
    q_t = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
    dout = torch.from_numpy(gb.view(np.int16)).cuda().view(torch.bfloat16)
    scale = 1.0 / np.sqrt(d)
    d_qoffs = torch.from_numpy(q_offsets).cuda()
    lse = torch.empty(T, hq, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(q_t, d_qoffs, kv_lens, cache, scale, max(q_lens), max_len, lse=lse)
    rows = int(offs[-1])
    dq, dk, dv = nk.ragged_paged_attention_backward(q_t, d_qoffs, kv_lens, cache, scale, max_len, out, dout, lse,
                                                    d_offs, rows)
    torch.cuda.synchronize()
    o_cache, o_table, kept = o_pack.attention_pack(k, v, offs, kept_in, "bf16", P)
    _, dk_o, dv_o = o_attn.ragged_paged_attention_backward(formats.bf16_value(qb), q_offsets, kept, o_cache,
                                                           o_table, scale, formats.bf16_value(gb), -1, 0, 0)
    dkg, dvg = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.all(np.isfinite(dkg)) and np.all(np.isfinite(dvg))
    for s in range(len(slots)):
        a, n = int(offs[s]), int(kept[s])
        sk = max(1.0, float(np.max(np.abs(dk_o[s])))) if n else 1.0
        sv = max(1.0, float(np.max(np.abs(dv_o[s])))) if n else 1.0
        gu.check_close(dkg[a:a + n] / sk, dk_o[s] / sk, 2e-2, f"dk segment {s}")
        gu.check_close(dvg[a:a + n] / sv, dv_o[s] / sv, 2e-2, f"dv segment {s}")
        assert np.all(dkg[a + n:int(offs[s + 1])] == 0.0) and np.all(dvg[a + n:int(offs[s + 1])] == 0.0)
