"""GPU parity of the fused RoPE + append on its own, over the whole cache.

V pages keep 4 consecutive slots of a dimension in one 16-byte run, so the
append writes whole slot quads where it can and single elements where a
segment's new slots start or end inside a quad.  These cases place new slots
at every offset inside a quad (segments of 1..13 new tokens after 0..93
cached ones, an empty segment, several segments inside one group of four
tokens) and compare every cache element -- appended and untouched, K, V and
e4m3 scales -- with the oracle's cache after its own append, bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

RAGGED = dict(q_lens=[1, 2, 3, 5, 7, 0, 9, 4, 13, 1], kv_lens=[3, 10, 3, 6, 100, 5, 9, 4, 40, 1])

CASES = {
    "bf16_d128_p16": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128),
    "e4m3_d128_p16": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, cache_dtype="e4m3"),
    "f32_d64_p32": dict(**RAGGED, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=32,
                        in_dtype="f32", cache_dtype="f32"),
    "bf16_d256_p32_interleaved": dict(q_lens=[5, 9, 2, 1], kv_lens=[9, 9, 70, 33], num_q_heads=4,
                                      num_kv_heads=2, head_dim=256, page_size=32, rope_layout="interleaved",
                                      rotary_dim=128),
    "e4m3_d64_p32_decode": dict(q_lens=[1] * 6, kv_lens=[1, 2, 3, 4, 5, 64], num_q_heads=4, num_kv_heads=1,
                                head_dim=64, page_size=32, cache_dtype="e4m3", explicit_positions=False),
    # p-RoPE: rotate-half pairs over the whole head, only the first rotated
    "bf16_d128_p16_proportional": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       rope_layout="half_proportional", rotary_dim=64),
    "e4m3_d256_p32_proportional": dict(q_lens=[5, 9, 2, 1], kv_lens=[9, 9, 70, 33], num_q_heads=4,
                                       num_kv_heads=2, head_dim=256, page_size=32, cache_dtype="e4m3",
                                       rope_layout="half_proportional", rotary_dim=64),
    "f32_d64_p16_proportional_full": dict(q_lens=[7, 3], kv_lens=[20, 3], num_q_heads=2, num_kv_heads=2,
                                          head_dim=64, in_dtype="f32", cache_dtype="f32",
                                          rope_layout="half_proportional", rotary_dim=64),
    # 136 heads x 8 units per token: a token's Q/K units span two work-groups
    "bf16_d128_hq128_two_blocks_per_token": dict(q_lens=[3, 6], kv_lens=[10, 6], num_q_heads=128,
                                                 num_kv_heads=8, head_dim=128),
}


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return (a == b) | (np.isnan(a) & np.isnan(b))


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_whole_cache(name):
    w = synth.custom(**CASES[name], name=name)
    gu.say(f"append {name}: T={w.total_q} B={w.num_seqs} D={w.head_dim} P={w.page_size} cache={w.cache_dtype}")
    d = gu.to_device(w)
    c = d["cache"]
    nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], c,
                           w.rotary_dim, w.rope_layout, position_ids=d["position_ids"])
    torch.cuda.synchronize()

    def raw(t):
        t = t.cpu()
        if w.cache_dtype == "f32":
            return t.numpy()
        if w.cache_dtype == "bf16":
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.view(torch.uint8).numpy()

    ks = None if c.k_scales is None else c.k_scales.cpu().numpy()
    vs = None if c.v_scales is None else c.v_scales.cpu().numpy()
    got = PagedCache.from_storage(w.cache_dtype, raw(c.k_pages), raw(c.v_pages), ks, vs)
    _, want, _, _ = gu.oracle_run(w, d["raw_cache"])
    for what, g, o in (("K", got.k, want.k), ("V", got.v, want.v)):
        ok = _same(g, o)
        assert ok.all(), f"{what}: {int((~ok).sum())} elements differ, first at {np.argwhere(~ok)[0].tolist()}"
    if w.cache_dtype == "e4m3":
        for what, g, o in (("K scales", got.k_scale, want.k_scale), ("V scales", got.v_scale, want.v_scale)):
            ok = _same(g, o)
            assert ok.all(), f"{what}: {int((~ok).sum())} differ, first at {np.argwhere(~ok)[0].tolist()}"
    gu.say(f"append {name}: whole cache bit-equal")
