"""GPU parity on shapes the oracle finishes in seconds but that span several
tiles, ragged tails, every head_dim / page size / dtype / RoPE layout the
library builds, windows, GQA ratios 1..32, split-KV chunking, and the edge
cases (empty batch, rows with no key, window of one key), plus bit-exact
invariants (determinism, page placement)."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import attention as o_attn
from oracle import formats, merge as o_merge
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = {
    # name: kwargs of synth.custom
    "prefill_ragged_d128": dict(q_lens=[1, 2, 33, 100, 257, 64], kv_lens=[1, 2, 33, 100, 257, 64],
                                num_q_heads=8, num_kv_heads=2, head_dim=128),
    "chunked_prefill_d64_p32_mha": dict(q_lens=[40, 70, 3], kv_lens=[300, 71, 50], num_q_heads=4,
                                        num_kv_heads=4, head_dim=64, page_size=32, rope_layout="interleaved",
                                        rotary_dim=32),
    "window_mixed_d256": dict(q_lens=[300, 1, 1, 129], kv_lens=[300, 1000, 60, 129], num_q_heads=4,
                              num_kv_heads=2, head_dim=256, page_size=32, rope_layout="interleaved",
                              rotary_dim=128, window_left=100, softmax_scale=1.0, qk_norm=True),
    "decode_lengths_g8": dict(q_lens=[1] * 9, kv_lens=[1, 31, 32, 33, 511, 512, 513, 2000, 4097],
                              num_q_heads=32, num_kv_heads=4, head_dim=128, explicit_positions=False),
    "decode_fp8_g8": dict(q_lens=[1] * 7, kv_lens=[1, 17, 64, 513, 1500, 4100, 9000], num_q_heads=64,
                          num_kv_heads=8, head_dim=128, cache_dtype="e4m3", explicit_positions=False,
                          split_tokens=512),
    "decode_g32_d64_p32": dict(q_lens=[1] * 4, kv_lens=[5, 200, 1025, 3000], num_q_heads=32,
                               num_kv_heads=1, head_dim=64, page_size=32),
    "decode_g16_d256_window": dict(q_lens=[1] * 3, kv_lens=[40, 2048, 5000], num_q_heads=32,
                                   num_kv_heads=2, head_dim=256, window_left=1023),
    "prefill_fp8_d128": dict(q_lens=[17, 40, 1], kv_lens=[17, 90, 300], num_q_heads=8, num_kv_heads=2,
                             head_dim=128, cache_dtype="e4m3"),
    "prefill_window0_d64": dict(q_lens=[50, 7], kv_lens=[50, 20], num_q_heads=2, num_kv_heads=1,
                                head_dim=64, window_left=0),
    "f32_mixed_d128_p32": dict(q_lens=[9, 1, 30], kv_lens=[9, 77, 45], num_q_heads=6, num_kv_heads=2,
                               head_dim=128, page_size=32, in_dtype="f32", cache_dtype="f32"),
    "prefill_g3_d128": dict(q_lens=[65, 2], kv_lens=[65, 2], num_q_heads=6, num_kv_heads=2, head_dim=128),
    # head_dim 256 work-groups: 1, 2 or 4 heads x 4, 2 or 1 row blocks x 2 output halves
    "prefill_d256_mha_p16": dict(q_lens=[150, 37], kv_lens=[150, 60], num_q_heads=2, num_kv_heads=2,
                                 head_dim=256),
    "prefill_d256_g8_fp8": dict(q_lens=[70, 5], kv_lens=[100, 5], num_q_heads=16, num_kv_heads=2,
                                head_dim=256, page_size=32, cache_dtype="e4m3"),
    # 8 query heads per work-group at head_dim 256: 16-row q-blocks, each segment ending in a partial one
    "prefill_d256_g8_ragged": dict(q_lens=[70, 5, 33, 16], kv_lens=[100, 5, 33, 80], num_q_heads=16,
                                   num_kv_heads=2, head_dim=256, page_size=32),
    # the largest query-head group a KV head may have (64): 4 blocks of 16 decode columns, 8 prefill heads
    # per work-group
    "max_group_g64_d128": dict(q_lens=[1, 40, 1], kv_lens=[700, 40, 33], num_q_heads=64, num_kv_heads=1,
                               head_dim=128),
    # 2100 short prefill segments, some over prior keys: more than the 2048 segments whose offsets the plan
    # kernel keeps in LDS, so the work list is built from the offsets in global memory
    "prefill_many_segments_d64": dict(q_lens=[2, 3, 5, 17] * 525,
                                      kv_lens=[q + (i % 3) * 7 for i, q in enumerate([2, 3, 5, 17] * 525)],
                                      num_q_heads=4, num_kv_heads=2, head_dim=64),
    # p-RoPE (a quarter of the pairs rotated) under a sliding window, decode rows included
    "proportional_rope_d256_window": dict(q_lens=[90, 1, 1], kv_lens=[90, 700, 40], num_q_heads=8,
                                          num_kv_heads=2, head_dim=256, page_size=32,
                                          rope_layout="half_proportional", rotary_dim=64, window_left=200,
                                          rope_theta=1e6),
}


def _run_and_compare(w, split=None):
    d = gu.to_device(w)
    q_out, out, lse = gu.run_hip(w, d, split=split)
    torch.cuda.synchronize()
    q_o, cache_o, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
    gu.compare_storage(gu.host_values(q_out, w.in_dtype), q_o, w.in_dtype, "q_out")
    tol = gu.tol_for(w)
    e1 = gu.check_close(gu.host_values(out, w.in_dtype), out_o, tol, "out")
    e2 = gu.check_close(lse.cpu().numpy(), lse_o, tol, "lse")
    return e1, e2, d, (q_out, out, lse)


@pytest.mark.parametrize("name", sorted(CASES))
def test_parity_case(name):
    w = synth.custom(**CASES[name], name=name)
    gu.say(f"case {name}: T={w.total_q} B={w.num_seqs} D={w.head_dim} P={w.page_size} "
           f"G={w.num_q_heads // w.num_kv_heads} cache={w.cache_dtype}")
    e1, e2, _, _ = _run_and_compare(w)
    gu.say(f"case {name}: out err {e1:.3g} lse err {e2:.3g}")
    gu.record_margin(f"parity {name}", e1, e2, gu.tol_for(w))


@pytest.mark.parametrize("split", [32, 96, 512, 0])
def test_decode_split_sizes(split):
    w = synth.custom(q_lens=[1] * 5, kv_lens=[1, 100, 777, 2048, 3333], num_q_heads=16, num_kv_heads=4,
                     head_dim=128, explicit_positions=False, name="split")
    gu.say(f"decode split {split}")
    _run_and_compare(w, split=split)


@pytest.mark.parametrize("split", [96, 512, 1024])
def test_decode_split_sizes_e4m3(split):
    """e4m3 decode: chunks of 16-step sub-chunks (split below 512), of one
    32-step sub-chunk, and of two (split 1024), each sub-chunk with its own
    scale loads."""
    w = synth.custom(q_lens=[1] * 5, kv_lens=[1, 100, 777, 2048, 3333], num_q_heads=16, num_kv_heads=4,
                     head_dim=128, cache_dtype="e4m3", explicit_positions=False, name="split_e4m3")
    gu.say(f"decode e4m3 split {split}")
    e1, e2, _, _ = _run_and_compare(w, split=split)
    gu.record_margin(f"parity decode_e4m3_split{split}", e1, e2, gu.tol_for(w))


def test_split_rows_reuse_workspace():
    """One workspace serves several split-KV calls in a row, including a call
    with fewer sequences and then one with the first call's shape again:
    every call's out and lse are bit-identical to a call on a fresh
    workspace (the workspace needs no initialisation between calls)."""
    big = synth.custom(q_lens=[1, 1, 1, 40, 1], kv_lens=[3000, 129, 4100, 40, 777], num_q_heads=32,
                       num_kv_heads=4, head_dim=128, split_tokens=64, name="reuse_big")
    small = synth.custom(q_lens=[1, 1], kv_lens=[2500, 65], num_q_heads=32, num_kv_heads=4, head_dim=128,
                         split_tokens=64, name="reuse_small")
    gu.say("split rows: workspace reuse")
    ws = None
    for w in (big, small, big, big):
        d = gu.to_device(w)
        q_out = nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"],
                                       d["cache"], w.rotary_dim, w.rope_layout, position_ids=d["position_ids"])
        need = nk.workspace_size(q_out.dtype, d["cache"], w.num_seqs, w.total_q, w.max_q_len, w.max_kv_len,
                                 w.num_q_heads, w.window_left, w.split_tokens)
        if ws is None:
            ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
        assert ws.numel() >= need
        args = (q_out, d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale, w.max_q_len, w.max_kv_len,
                w.window_left)
        lse_a = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
        out_a, _ = nk.ragged_paged_attention(*args, lse=lse_a, kv_split_tokens=w.split_tokens, workspace=ws)
        lse_b = torch.empty_like(lse_a)
        out_b, _ = nk.ragged_paged_attention(*args, lse=lse_b, kv_split_tokens=w.split_tokens)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        assert np.array_equal(lse_a.cpu().numpy(), lse_b.cpu().numpy())
        _, _, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
        gu.check_close(gu.host_values(out_a, "bf16"), out_o, 2e-2, "out")
        gu.check_close(lse_a.cpu().numpy(), lse_o, 2e-2, "lse")


def test_deterministic_and_page_placement_invariant():
    base = dict(q_lens=[1, 1, 200], kv_lens=[900, 33, 260], num_q_heads=8, num_kv_heads=2, head_dim=128)
    w1 = synth.custom(**base, seed=1)
    # same values, other physical pages: relabel every physical page
    perm = np.random.default_rng(77).permutation(w1.num_pages).astype(np.int32)
    w2 = dataclasses.replace(w1, page_table=perm[w1.page_table])
    assert not np.array_equal(w1.page_table, w2.page_table)
    gu.say("determinism / page placement")
    outs = []
    for w in (w1, w1, w2):
        d = gu.to_device(w)
        q_out, out, lse = gu.run_hip(w, d)
        torch.cuda.synchronize()
        outs.append((q_out.cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_future_keys_do_not_matter():
    """Overwrite the cache slots after each prefill row's position: rows
    before them are bit-identical."""
    w = synth.custom(q_lens=[150], kv_lens=[150], num_q_heads=4, num_kv_heads=2, head_dim=128, page_order="in_order")
    gu.say("future-key perturbation")
    d = gu.to_device(w)
    q_out, out, lse = gu.run_hip(w, d)
    torch.cuda.synchronize()
    ref = out.clone()
    c = d["cache"]
    # scramble keys 100.. (pages 6..): rows 0..99 must not change
    c.k_pages[6:] = torch.randn_like(c.k_pages[6:].float()).to(c.k_pages.dtype)
    c.v_pages[6:] = torch.randn_like(c.v_pages[6:].float()).to(c.v_pages.dtype)
    # the rows sitting at positions < 96 only see pages 0..5
    out2, _ = nk.ragged_paged_attention(q_out, d["q_offsets"], d["kv_lens"], c, w.softmax_scale, w.max_q_len,
                                        w.max_kv_len, w.window_left)
    torch.cuda.synchronize()
    assert torch.equal(out2[:96].view(torch.int16), ref[:96].view(torch.int16))
    assert not torch.equal(out2[100:].view(torch.int16), ref[100:].view(torch.int16))


def test_rows_without_keys_and_empty_segments():
    """q_len > kv_len (rows before the first key) give zeros and -inf; empty
    segments are skipped; attention alone on a generated cache."""
    w = synth.custom(q_lens=[5, 0, 1, 40], kv_lens=[3, 0, 0, 40], num_q_heads=4, num_kv_heads=2, head_dim=64)
    gu.say("rows without keys")
    raw = synth.build_cache(w)
    d = gu.to_device(w, cache=raw)
    # fill the fresh segment's keys directly (no RoPE step: q_len > kv_len is
    # outside the append's precondition)
    rng = np.random.default_rng(5)
    kp = d["cache"].k_pages
    kp.copy_(torch.from_numpy(rng.standard_normal(tuple(kp.shape), dtype=np.float32)).to(kp))
    vp = d["cache"].v_pages
    vp.copy_(torch.from_numpy(rng.standard_normal(tuple(vp.shape), dtype=np.float32)).to(vp))
    lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
    out, lse = nk.ragged_paged_attention(d["q"], d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale,
                                         w.max_q_len, w.max_kv_len, w.window_left, lse=lse)
    torch.cuda.synchronize()
    cache_o = PagedCache.from_storage("bf16", kp.cpu().view(torch.int16).numpy().view(np.uint16),
                                      vp.cpu().view(torch.int16).numpy().view(np.uint16))
    q = formats.bf16_value(d["tokens"]["q"])
    out_o, lse_o = o_attn.ragged_paged_attention(q, w.q_offsets, w.kv_lens, cache_o, w.page_table,
                                                 w.softmax_scale, w.window_left)
    og = gu.host_values(out, "bf16")
    gu.check_close(og, out_o, 2e-2, "out")
    gu.check_close(lse.cpu().numpy(), lse_o, 2e-2, "lse")
    assert np.all(og[:2] == 0) and np.all(np.isneginf(lse.cpu().numpy()[:2]))
    assert np.all(og[5] == 0) and np.all(np.isneginf(lse.cpu().numpy()[5]))   # kv_len 0 decode row


def test_empty_batch_is_a_no_op():
    w = synth.custom(q_lens=[3], kv_lens=[3], num_q_heads=2, num_kv_heads=1, head_dim=64)
    d = gu.to_device(w)
    q = d["q"][:0]
    offs = torch.zeros(2, dtype=torch.int32, device="cuda")
    out, _ = nk.ragged_paged_attention(q, offs, d["kv_lens"], d["cache"], 0.1, 0, 3)
    assert out.shape[0] == 0


@pytest.mark.parametrize("D", [128, 64, 130, 256, 512])
def test_lse_merge_entry_point(D):
    rng = np.random.default_rng(7)
    n, H = 93, 5
    po = rng.standard_normal((n, H, D)).astype(np.float32)
    pl = (rng.standard_normal((n, H)) * 4).astype(np.float32)
    pl[3, 2] = -np.inf
    pl[10:12, :] = -np.inf
    # an empty row, an all -inf row, and a row of 70 chunks (more than a wave's lanes)
    offs = np.array([0, 3, 3, 10, 12, 23, 93], dtype=np.int32)
    gu.say(f"lse merge entry point, head_dim {D}")
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty(len(offs) - 1, H, D, dtype=dt, device="cuda")
        lse = torch.empty(len(offs) - 1, H, dtype=torch.float32, device="cuda")
        nk.attention_lse_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                               torch.from_numpy(offs).cuda(), out, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = o_merge.lse_merge(po, pl, offs)
        tol = 1e-5 if dt == torch.float32 else 2e-2
        gu.check_close(out.float().cpu().numpy(), ref_o, tol, "merge out")
        gu.check_close(lse.cpu().numpy(), ref_l, 1e-5, "merge lse")
        assert np.all(np.isneginf(lse.cpu().numpy()[1])) and np.all(lse.cpu().numpy()[3] == -np.inf)
