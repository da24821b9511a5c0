"""The allocation-free attention entry point (nk_ragged_paged_attention_noalloc,
for callers that cannot allocate) against the workspace entry point
(nk_ragged_paged_attention_band): the same kernels on the same inputs, so out
and lse must be bit-identical, and within the oracle's tolerance.  Two calls
in a row, the second on a smaller batch, so that the second reuses the
static scratch the first left behind."""

import numpy as np
import pytest
import torch

import synth
from ragged_paged_kv_amd import nk
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# a mixed batch (prefill segments, decode rows spanning many split-KV chunks)
# and a smaller one after it
CALLS = [
    ("first", dict(q_lens=[70, 1, 130, 1, 1, 33, 1], kv_lens=[70, 3000, 200, 900, 4100, 90, 77], num_q_heads=16,
                   num_kv_heads=4, head_dim=128, split_tokens=64)),
    ("second_smaller", dict(q_lens=[1, 20, 1], kv_lens=[700, 20, 1500], num_q_heads=16, num_kv_heads=4,
                            head_dim=128, split_tokens=64)),
]


def _compare(name, spec):
    w = synth.custom(**spec, name=name)
    gu.say(f"noalloc {name}: B={w.num_seqs} T={w.total_q} max_kv={w.max_kv_len} split={w.split_tokens}")
    d = gu.to_device(w)
    q_out = nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"], d["cache"],
                                   w.rotary_dim, w.rope_layout, position_ids=d["position_ids"])
    need = nk.workspace_size(q_out.dtype, d["cache"], w.num_seqs, w.total_q, w.max_q_len, w.max_kv_len,
                             w.num_q_heads, w.window_left, w.split_tokens)
    assert 0 < need <= nk.NOALLOC_SCRATCH_BYTES
    args = (q_out, d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale, w.max_q_len, w.max_kv_len,
            w.window_left)
    lse_a = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device="cuda")
    out_a, _ = nk.ragged_paged_attention(*args, lse=lse_a, kv_split_tokens=w.split_tokens)
    lse_b = torch.empty_like(lse_a)
    out_b, _ = nk.ragged_paged_attention_noalloc(*args, lse=lse_b, kv_split_tokens=w.split_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "out differs from the workspace call"
    la, lb = lse_a.cpu().numpy(), lse_b.cpu().numpy()
    assert np.array_equal(la, lb), "lse differs from the workspace call"
    _, _, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
    tol = gu.tol_for(w)
    e1 = gu.check_close(gu.host_values(out_b, w.in_dtype), out_o, tol, "out")
    e2 = gu.check_close(lb, lse_o, tol, "lse")
    gu.say(f"noalloc {name}: bit-identical to the workspace call; out err {e1:.3g} lse err {e2:.3g}")


def test_noalloc_matches_workspace_call_twice():
    for name, spec in CALLS:
        _compare(name, spec)
