"""GPU parity of the general band of keys (nk_ragged_paged_attention_band):
the row at position p sees keys p - window_left .. p + window_right, -1
standing for an unbounded side (NumKong matrix-kernels page,
attention_packed).  Prefill rows see keys after their own position, up to
the whole segment; single-token rows sit at their segment's last key and
are unchanged; rows placed before the segment's first key (more new rows
than keys) can reach keys through the band's right side.  Same tolerances
as the causal cases, against the oracle's float64 values."""

import numpy as np
import pytest
import torch

import synth
from oracle import attention as o_attn
from oracle import formats
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

RAGGED = dict(q_lens=[70, 130, 1, 33], kv_lens=[70, 200, 50, 90])

CASES = {
    "after3_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, window_right=3),
    "after70_window40_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                       window_left=40, window_right=70),
    "bidirectional_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, window_right=-1),
    "after5_e4m3_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, cache_dtype="e4m3",
                             window_right=5),
    "after9_window20_bf16_d256_p32": dict(q_lens=[90, 1, 40], kv_lens=[90, 300, 100], num_q_heads=4,
                                          num_kv_heads=2, head_dim=256, page_size=32, rope_layout="interleaved",
                                          rotary_dim=128, window_left=20, window_right=9),
    "bidirectional_d64_p32_mha": dict(q_lens=[64, 65], kv_lens=[64, 65], num_q_heads=4, num_kv_heads=4,
                                      head_dim=64, page_size=32, window_right=-1),
    "after2_f32_d64": dict(q_lens=[9, 30, 1], kv_lens=[9, 45, 12], num_q_heads=4, num_kv_heads=2, head_dim=64,
                           in_dtype="f32", cache_dtype="f32", window_right=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_band_parity(name):
    w = synth.custom(**CASES[name], name=name)
    gu.say(f"band {name}: T={w.total_q} B={w.num_seqs} D={w.head_dim} window=({w.window_left}, {w.window_right}) "
           f"cache={w.cache_dtype}")
    d = gu.to_device(w)
    q_out, out, lse = gu.run_hip(w, d)
    torch.cuda.synchronize()
    _, _, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
    tol = gu.tol_for(w)
    e1 = gu.check_close(gu.host_values(out, w.in_dtype), out_o, tol, "out")
    e2 = gu.check_close(lse.cpu().numpy(), lse_o, tol, "lse")
    gu.say(f"band {name}: out err {e1:.3g} lse err {e2:.3g}")
    gu.record_margin(f"band {name}", e1, e2, gu.tol_for(w))


def test_band_zero_is_causal_bit_for_bit():
    """window_right = 0 through the band entry point is the causal call."""
    w = synth.custom(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, name="band_zero")
    gu.say("band zero vs causal")
    d = gu.to_device(w)
    _, out_b, lse_b = gu.run_hip(w, d)                     # window_right 0 (the band entry point)
    torch.cuda.synchronize()
    from ragged_paged_kv_amd import nk
    import ctypes
    c = d["cache"].struct()
    q_out = nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], d["cache"],
                                   w.rotary_dim, w.rope_layout, position_ids=d["position_ids"])
    out_c = torch.empty_like(q_out)
    lse_c = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
    need = nk.workspace_size(q_out.dtype, d["cache"], w.num_seqs, w.total_q, w.max_q_len, w.max_kv_len,
                             w.num_q_heads, w.window_left, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = nk.lib().nk_ragged_paged_attention(
        q_out.data_ptr(), nk.NK_BF16, d["q_offsets"].data_ptr(), d["kv_lens"].data_ptr(), ctypes.byref(c),
        float(w.softmax_scale), int(w.window_left), out_c.data_ptr(), lse_c.data_ptr(), w.num_seqs, w.total_q,
        w.max_q_len, w.max_kv_len, w.num_q_heads, 0, ws.data_ptr(), ws.numel(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nk.NK_OK
    torch.cuda.synchronize()
    assert torch.equal(out_b.view(torch.int16), out_c.view(torch.int16))
    assert np.array_equal(lse_b.cpu().numpy(), lse_c.cpu().numpy())


@pytest.mark.parametrize("after", [5, 8, 10, -1])
def test_band_rows_before_keys(after):
    """20 new rows over 8 keys: rows 0..11 sit before the first key (outside
    the append's precondition, so attention alone on a generated cache).
    With keys after their position they reach the first keys (rows 7..11 with
    5 after, 4..11 with 8 and 2..11 with 10: a right side as long as the
    segment or longer still starts at the row's own position); with an
    unbounded right side every row sees all 8."""
    w = synth.custom(q_lens=[20, 3], kv_lens=[8, 40], num_q_heads=2, num_kv_heads=1, head_dim=64,
                     window_right=after, name="band_rows_before_keys")
    gu.say(f"band rows before keys, after={after}")
    d = gu.to_device(w)
    rng = np.random.default_rng(6)
    kp, vp = d["cache"].k_pages, d["cache"].v_pages
    kp.copy_(torch.from_numpy(rng.standard_normal(tuple(kp.shape), dtype=np.float32)).to(kp))
    vp.copy_(torch.from_numpy(rng.standard_normal(tuple(vp.shape), dtype=np.float32)).to(vp))
    lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(d["q"], d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale,
                                         w.max_q_len, w.max_kv_len, w.window_left, lse=lse, window_right=after)
    torch.cuda.synchronize()
    cache_o = PagedCache.from_storage("bf16", kp.cpu().view(torch.int16).numpy().view(np.uint16),
                                      vp.cpu().view(torch.int16).numpy().view(np.uint16))
    q = formats.bf16_value(d["tokens"]["q"])
    out_o, lse_o = o_attn.ragged_paged_attention(q, w.q_offsets, w.kv_lens, cache_o, w.page_table,
                                                 w.softmax_scale, w.window_left, window_right=after)
    og = gu.host_values(out, "bf16")
    gu.check_close(og, out_o, 2e-2, "out")
    gu.check_close(lse.cpu().numpy(), lse_o, 2e-2, "lse")
    lg = lse.cpu().numpy()
    first_seen = 0 if after < 0 else max(0, 12 - after)  # first row whose band reaches key 0
    assert np.all(np.isneginf(lg[:first_seen])) and np.all(og[:first_seen] == 0)
    assert np.all(np.isfinite(lg[first_seen:20]))
