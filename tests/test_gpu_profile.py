"""GPU checks of the kernel-timing diagnostics (nk_profile_*).

The timing events ride on the kernels' own dispatches (hipExtLaunchKernel),
so these cases check that a selected family reports one timed launch per
call with a positive duration, that unselected families and disabled timing
report none, that reset clears the totals, and that timing does not change
a single output bit.
"""

import numpy as np
import pytest
import torch

import synth
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(w, d, out, lse):
    c = d["cache"]
    nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], c,
                           w.rotary_dim, w.rope_layout, position_ids=d["position_ids"], q_out=d["q_out"])
    nk.ragged_paged_attention(d["q_out"], d["q_offsets"], d["kv_lens"], c, w.softmax_scale, w.max_q_len,
                              w.max_kv_len, w.window_left, out=out, lse=lse, kv_split_tokens=w.split_tokens)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_profile_counts_and_outputs(kind):
    if kind == "decode":      # several chunks per row: decode kernel and merge
        w = synth.custom(q_lens=[1] * 6, kv_lens=[40, 300, 700, 5, 1000, 64], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, split_tokens=128, name="profile_decode")
        fam = "attn_decode"
    else:                     # the prefill scope holds its plan kernel and the prefill kernel
        w = synth.custom(q_lens=[70, 130], kv_lens=[70, 200], num_q_heads=8, num_kv_heads=2, head_dim=128,
                         name="profile_prefill")
        fam = "attn_prefill"
    gu.say(f"profile {kind}: T={w.total_q} B={w.num_seqs}")
    raw = synth.build_cache(w)

    def fresh():
        d = gu.to_device(w, cache=raw)
        d["q_out"] = torch.empty_like(d["q"])
        out = torch.empty_like(d["q"])
        lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
        return d, out, lse

    d, out0, lse0 = fresh()
    nk.profile_enable(False)
    nk.profile_reset()
    _run(w, d, out0, lse0)
    torch.cuda.synchronize()
    assert nk.profile_read(fam) == (0.0, 0)                  # timing off: nothing recorded

    d, out1, lse1 = fresh()
    nk.profile_enable(True, [fam])
    try:
        _run(w, d, out1, lse1)
        torch.cuda.synchronize()
        ms, n = nk.profile_read(fam)
        assert n == 1 and 0.0 < ms < 1000.0, (ms, n)
        assert nk.profile_read("rope_write") == (0.0, 0)     # not selected
        if kind == "decode":
            assert nk.profile_read("lse_merge") == (0.0, 0)
            nk.profile_enable(True, ["attn_decode", "lse_merge"])
            _run(w, d, out1, lse1)
            torch.cuda.synchronize()
            assert nk.profile_read("attn_decode")[1] == 2 and nk.profile_read("lse_merge")[1] == 1
        nk.profile_reset()
        assert nk.profile_read(fam) == (0.0, 0)
    finally:
        nk.profile_enable(False)
    # timed and untimed runs write the same bits
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert np.array_equal(lse0.cpu().numpy(), lse1.cpu().numpy())


def test_prefill_only_batch_launches_no_decode_kernel():
    """With min_q_len >= 2 (a batch without single-token rows) the call
    launches no decode or merge kernel, and its outputs are bit-identical to
    the call that does not state the bound."""
    w = synth.custom(q_lens=[70, 130, 33], kv_lens=[70, 200, 90], num_q_heads=8, num_kv_heads=2, head_dim=128,
                     name="prefill_only")
    gu.say("prefill-only batch: launches")
    d = gu.to_device(w)
    d["q_out"] = torch.empty_like(d["q"])
    c = d["cache"]
    nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], c, w.rotary_dim,
                           w.rope_layout, position_ids=d["position_ids"], q_out=d["q_out"])
    outs = []
    try:
        for min_q in (0, int(w.q_lens.min())):
            nk.profile_reset()
            nk.profile_enable(True)
            out = torch.empty_like(d["q"])
            lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
            nk.ragged_paged_attention(d["q_out"], d["q_offsets"], d["kv_lens"], c, w.softmax_scale, w.max_q_len,
                                      w.max_kv_len, w.window_left, out=out, lse=lse, min_q_len=min_q)
            torch.cuda.synchronize()
            outs.append((out, lse, nk.profile_read("attn_decode")[1], nk.profile_read("attn_prefill")[1]))
    finally:
        nk.profile_enable(False)
    assert outs[0][2] == 1 and outs[1][2] == 0          # the decode launch only without the bound
    assert outs[0][3] == 1 and outs[1][3] == 1
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert np.array_equal(outs[0][1].cpu().numpy(), outs[1][1].cpu().numpy())
