"""GPU parity of M-RoPE (nk_rope_qk_write_paged_mrope): the rotated pairs
split into sections, each rotated by its own position stream (Mojo page,
mrope_section).  Three streams in the manner of vision-language models
(temporal, height, width); q_out and every cache element -- K, V and e4m3
scales -- bit-equal to the oracle's fused step."""

import numpy as np
import pytest
import torch

import synth
from oracle import rope as o_rope
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = {
    "half_bf16_d128_16_24_24": dict(layout="half", head_dim=128, rotary_dim=128, sections=[16, 24, 24],
                                    cache_dtype="bf16"),
    "interleaved_e4m3_d128_24_8_32": dict(layout="interleaved", head_dim=128, rotary_dim=128, sections=[24, 8, 32],
                                          cache_dtype="e4m3"),
    "proportional_bf16_d256_p32_8_16_8": dict(layout="half_proportional", head_dim=256, rotary_dim=64,
                                              sections=[8, 16, 8], cache_dtype="bf16", page_size=32),
    "half_f32_d64_one_section": dict(layout="half", head_dim=64, rotary_dim=64, sections=[32], cache_dtype="f32",
                                     in_dtype="f32"),
}


def _streams(w):
    """Per token: temporal = its slot; height and width walk a 4-wide grid."""
    slots = w.positions.astype(np.int64)
    return np.stack([slots, slots // 4, slots % 4 + slots // 16]).astype(np.int32)


@pytest.mark.parametrize("name", sorted(CASES))
def test_mrope_append_and_q(name):
    c = CASES[name]
    w = synth.custom(q_lens=[5, 9, 1, 13], kv_lens=[20, 9, 40, 77], num_q_heads=4, num_kv_heads=2,
                     head_dim=c["head_dim"], rotary_dim=c["rotary_dim"], rope_layout=c["layout"],
                     page_size=c.get("page_size", 16), in_dtype=c.get("in_dtype", "bf16"),
                     cache_dtype=c["cache_dtype"], name=name)
    sections = c["sections"]
    pos = _streams(w)[:len(sections)] if len(sections) > 1 else _streams(w)[:1]
    gu.say(f"mrope {name}: T={w.total_q} sections={sections}")
    d = gu.to_device(w)
    cache = d["cache"]
    q_out = nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], cache,
                                   w.rotary_dim, w.rope_layout, position_ids=torch.from_numpy(pos).cuda(),
                                   mrope_sections=sections)
    torch.cuda.synchronize()

    nt = d["tokens"]
    conv = (lambda a: a.astype(np.float64)) if w.in_dtype == "f32" else gu.formats.bf16_value
    raw = d["raw_cache"]
    cache_o = PagedCache.from_storage(w.cache_dtype, raw["k_pages"], raw["v_pages"], raw["k_scales"], raw["v_scales"])
    q_o, cache2 = o_rope.rope_qk_write_paged(conv(nt["q"]), conv(nt["k"]), conv(nt["v"]), w.in_dtype, w.q_offsets,
                                             w.kv_lens, pos, synth.freqs_table(w), w.rotary_dim, w.rope_layout,
                                             cache_o, w.page_table, mrope_sections=sections)
    gu.compare_storage(gu.host_values(q_out, w.in_dtype), q_o, w.in_dtype, "q_out")

    def raw_of(t):
        t = t.cpu()
        if w.cache_dtype == "f32":
            return t.numpy()
        if w.cache_dtype == "bf16":
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.view(torch.uint8).numpy()
    ks = None if cache.k_scales is None else cache.k_scales.cpu().numpy()
    vs = None if cache.v_scales is None else cache.v_scales.cpu().numpy()
    got = PagedCache.from_storage(w.cache_dtype, raw_of(cache.k_pages), raw_of(cache.v_pages), ks, vs)
    for what, g, o in (("K", got.k, cache2.k), ("V", got.v, cache2.v)):
        same = (g == o) | (np.isnan(g) & np.isnan(o))
        assert same.all(), f"{what}: {int((~same).sum())} elements differ"
    if w.cache_dtype == "e4m3":
        for what, g, o in (("K scales", got.k_scale, cache2.k_scale), ("V scales", got.v_scale, cache2.v_scale)):
            same = (g == o) | (np.isnan(g) & np.isnan(o))
            assert same.all(), f"{what}: {int((~same).sum())} differ"
    gu.say(f"mrope {name}: q_out and cache bit-equal")
