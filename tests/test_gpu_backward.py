"""GPU parity of nk_ragged_paged_attention_backward (NumKong matrix-kernels
page, attention_packed_gradients): the GPU forward's out and lse, an output
gradient, then dq, dk, dv on the GPU against the oracle's gradients computed
from the plain definition in float64.  The GPU gradients read the forward's
stored (bf16) output and its float32 lse, so the bound is relative to the
gradients' scale: 2e-2 for bf16 inputs, 1e-4 for float32.  bf16 at head
dims 64 and 128 runs the MFMA kernels (P and dS rounded to bf16 for their
products), other head dims the float32 VALU kernels."""

import numpy as np
import pytest
import torch

import synth
from oracle import attention as o_attn
from oracle import formats
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

RAGGED = dict(q_lens=[70, 130, 1, 33], kv_lens=[70, 200, 50, 90])

CASES = {
    "causal_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128),
    "window40_sinks4_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128, window_left=40,
                                      sink_keys=4),
    "after5_bf16_d256_p32": dict(q_lens=[90, 1, 40], kv_lens=[90, 300, 100], num_q_heads=4, num_kv_heads=2,
                                 head_dim=256, page_size=32, rope_layout="interleaved", rotary_dim=128,
                                 window_right=5),
    "decode_gqa8_bf16_d64": dict(q_lens=[1, 1, 1], kv_lens=[500, 33, 129], num_q_heads=16, num_kv_heads=2,
                                 head_dim=64),
    "causal_f32_d64": dict(q_lens=[9, 30, 1], kv_lens=[9, 45, 12], num_q_heads=4, num_kv_heads=2, head_dim=64,
                           in_dtype="f32", cache_dtype="f32"),
    # MFMA path: several 128-key and 32-row tiles per segment, ragged tails,
    # 1, 2 and 4 query heads per KV head
    "long_causal_bf16_d128_g4": dict(q_lens=[300, 520, 1], kv_lens=[300, 600, 77], num_q_heads=16, num_kv_heads=4,
                                     head_dim=128),
    "window100_after7_bf16_d64_p32_g2": dict(q_lens=[260, 3, 190], kv_lens=[400, 3, 190], num_q_heads=4,
                                             num_kv_heads=2, head_dim=64, page_size=32, window_left=100,
                                             window_right=7),
    "window60_sinks8_bf16_d128_mha": dict(q_lens=[150, 150], kv_lens=[150, 300], num_q_heads=2, num_kv_heads=2,
                                          head_dim=128, window_left=60, sink_keys=8),
    # one query head per KV head at head_dim 64 (dK/dV written directly)
    "mha_bf16_d64_p16": dict(q_lens=[100, 64], kv_lens=[100, 130], num_q_heads=2, num_kv_heads=2, head_dim=64),
    # 16 query heads per KV head: 4 head chunks of 4 adding into dK/dV
    "causal_bf16_d64_g16": dict(q_lens=[200, 45], kv_lens=[260, 45], num_q_heads=32, num_kv_heads=2, head_dim=64,
                                page_size=32),
}


def _scaled_check(g, r, tol, what):
    s = max(1.0, float(np.max(np.abs(r))) if r.size else 1.0)
    return gu.check_close(np.asarray(g) / s, np.asarray(r) / s, tol, what)


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    w = synth.custom(**CASES[name], name=name)
    gu.say(f"backward {name}: T={w.total_q} B={w.num_seqs} D={w.head_dim} window=({w.window_left}, "
           f"{w.window_right}) sinks={w.sink_keys} in={w.in_dtype}")
    d = gu.to_device(w)
    q_out, out, lse = gu.run_hip(w, d)
    rng = np.random.default_rng(99)
    g = rng.standard_normal((w.total_q, w.num_q_heads, w.head_dim))
    if w.in_dtype == "f32":
        g = formats.f32_round(g)
        dout = torch.from_numpy(g.astype(np.float32)).cuda()
    else:
        gb = formats.bf16_bits(formats.bf16_round(g))
        g = formats.bf16_value(gb)
        dout = torch.from_numpy(gb.view(np.int16)).cuda().view(torch.bfloat16)
    key_offsets = np.concatenate([[0], np.cumsum(w.kv_lens)]).astype(np.int32)
    rows = int(key_offsets[-1])
    dq, dk, dv = nk.ragged_paged_attention_backward(
        q_out, d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale, w.max_kv_len, out, dout, lse,
        torch.from_numpy(key_offsets).cuda(), rows, w.window_left, w.window_right, w.sink_keys)
    torch.cuda.synchronize()

    q_o, cache_o, _, _ = gu.oracle_run(w, d["raw_cache"])
    dq_o, dk_o, dv_o = o_attn.ragged_paged_attention_backward(q_o, w.q_offsets, w.kv_lens, cache_o, w.page_table,
                                                              w.softmax_scale, g, w.window_left, w.window_right,
                                                              w.sink_keys)
    tol = 1e-4 if w.in_dtype == "f32" else 2e-2
    e1 = _scaled_check(dq.cpu().numpy(), dq_o, tol, "dq")
    dkg, dvg = dk.cpu().numpy(), dv.cpu().numpy()
    dk_ref = np.concatenate(dk_o, axis=0)
    dv_ref = np.concatenate(dv_o, axis=0)
    e2 = _scaled_check(dkg, dk_ref, tol, "dk")
    e3 = _scaled_check(dvg, dv_ref, tol, "dv")
    gu.say(f"backward {name}: scaled errors dq {e1:.3g} dk {e2:.3g} dv {e3:.3g}")


@pytest.mark.parametrize("after", [3, 10])
def test_backward_rows_before_keys(after):
    """Gradients with rows placed before the segment's first key (20 rows
    over 8 keys): a row reaches keys only through its band's right side,
    which starts at its own position also when it is as long as the segment
    or longer (10 after: rows 2..11 see a prefix of the keys, rows 0, 1 none
    and have zero dq)."""
    w = synth.custom(q_lens=[20, 3], kv_lens=[8, 40], num_q_heads=4, num_kv_heads=2, head_dim=64,
                     window_right=after, name="backward_rows_before_keys")
    gu.say(f"backward rows before keys, after={after}")
    d = gu.to_device(w)
    rng = np.random.default_rng(8)
    kp, vp = d["cache"].k_pages, d["cache"].v_pages
    kp.copy_(torch.from_numpy(rng.standard_normal(tuple(kp.shape), dtype=np.float32)).to(kp))
    vp.copy_(torch.from_numpy(rng.standard_normal(tuple(vp.shape), dtype=np.float32)).to(vp))
    lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(d["q"], d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale,
                                         w.max_q_len, w.max_kv_len, w.window_left, lse=lse, window_right=after)
    gb = formats.bf16_bits(formats.bf16_round(rng.standard_normal((w.total_q, w.num_q_heads, w.head_dim))))
    dout = torch.from_numpy(gb.view(np.int16)).cuda().view(torch.bfloat16)
    key_offsets = np.concatenate([[0], np.cumsum(w.kv_lens)]).astype(np.int32)
    rows = int(key_offsets[-1])
    dq, dk, dv = nk.ragged_paged_attention_backward(
        d["q"], d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale, w.max_kv_len, out, dout, lse,
        torch.from_numpy(key_offsets).cuda(), rows, w.window_left, after, 0)
    torch.cuda.synchronize()
    from oracle.paged import PagedCache
    cache_o = PagedCache.from_storage("bf16", kp.cpu().view(torch.int16).numpy().view(np.uint16),
                                      vp.cpu().view(torch.int16).numpy().view(np.uint16))
    q = formats.bf16_value(d["tokens"]["q"])
    dq_o, dk_o, dv_o = o_attn.ragged_paged_attention_backward(q, w.q_offsets, w.kv_lens, cache_o, w.page_table,
                                                              w.softmax_scale, formats.bf16_value(gb),
                                                              w.window_left, after, 0)
    dqg = dq.cpu().numpy()
    _scaled_check(dqg, dq_o, 2e-2, "dq")
    _scaled_check(dk.cpu().numpy(), np.concatenate(dk_o, axis=0), 2e-2, "dk")
    _scaled_check(dv.cpu().numpy(), np.concatenate(dv_o, axis=0), 2e-2, "dv")
    first_seen = max(0, 12 - after)
    assert np.all(dqg[:first_seen] == 0.0)
