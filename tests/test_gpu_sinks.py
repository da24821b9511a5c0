"""GPU parity of attention sinks beside a window (Algenta, "Ten named
techniques, one scalar formula each", streaming_llm_sink_score:
StreamingLLM keeps a segment's first keys visible beside the recent ones).
A row sees its band [p - window_left, p + window_right] and the keys
0 .. sink_keys-1 that are not right of the band.  Decode rows take the sink
keys as a split-KV chunk of their own; prefill work items visit the sink
keys' tiles before the band's.  Same tolerances as the causal cases, against
the oracle's float64 values."""

import numpy as np
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# decode rows far past the window (a sink chunk), prefill rows whose window
# starts inside and past the sink keys, a short segment the sinks cover whole
RAGGED = dict(q_lens=[70, 130, 1, 1, 33], kv_lens=[70, 200, 700, 50, 90])

CASES = {
    "sinks4_window40_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                      window_left=40, sink_keys=4),
    # sink keys over two tiles, overlapping the band of the early rows
    "sinks100_window40_bf16_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                        window_left=40, sink_keys=100),
    "sinks4_window40_e4m3_d128": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                      cache_dtype="e4m3", window_left=40, sink_keys=4),
    "sinks8_window20_after9_bf16_d256_p32": dict(q_lens=[90, 1, 40], kv_lens=[90, 300, 100], num_q_heads=4,
                                                 num_kv_heads=2, head_dim=256, page_size=32,
                                                 rope_layout="interleaved", rotary_dim=128, window_left=20,
                                                 window_right=9, sink_keys=8),
    # e4m3 at head_dim 256 (16-row waves, 4 heads per work-group), page 16
    "sinks4_window40_e4m3_d256_g4": dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=256,
                                         cache_dtype="e4m3", window_left=40, sink_keys=4),
    "sinks4_window64_gqa16_d64_p32": dict(q_lens=[1, 1, 200], kv_lens=[1000, 33, 260], num_q_heads=16,
                                          num_kv_heads=1, head_dim=64, page_size=32, window_left=64,
                                          sink_keys=4),
    "sinks4_window16_f32_d64": dict(q_lens=[9, 30, 1], kv_lens=[9, 45, 120], num_q_heads=4, num_kv_heads=2,
                                    head_dim=64, in_dtype="f32", cache_dtype="f32", window_left=16,
                                    sink_keys=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sink_parity(name):
    w = synth.custom(**CASES[name], name=name)
    gu.say(f"sinks {name}: T={w.total_q} B={w.num_seqs} D={w.head_dim} window=({w.window_left}, "
           f"{w.window_right}) sinks={w.sink_keys} cache={w.cache_dtype}")
    d = gu.to_device(w)
    _, out, lse = gu.run_hip(w, d)
    torch.cuda.synchronize()
    _, _, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
    tol = gu.tol_for(w)
    e1 = gu.check_close(gu.host_values(out, w.in_dtype), out_o, tol, "out")
    e2 = gu.check_close(lse.cpu().numpy(), lse_o, tol, "lse")
    gu.say(f"sinks {name}: out err {e1:.3g} lse err {e2:.3g}")
    gu.record_margin(f"sinks {name}", e1, e2, gu.tol_for(w))


@pytest.mark.parametrize("split", [128, 256])
def test_sink_chunk_with_many_band_chunks(split):
    """Decode rows whose window spans several split-KV chunks, plus the sink
    chunk; the merge combines all of them."""
    w = synth.custom(q_lens=[1, 1, 1, 1], kv_lens=[3000, 900, 40, 1500], num_q_heads=8, num_kv_heads=2,
                     head_dim=128, window_left=600, sink_keys=4, split_tokens=split, name="sinks_many_chunks")
    gu.say(f"sinks many chunks: split={split}")
    d = gu.to_device(w)
    _, out, lse = gu.run_hip(w, d)
    torch.cuda.synchronize()
    _, _, out_o, lse_o = gu.oracle_run(w, d["raw_cache"])
    gu.check_close(gu.host_values(out, "bf16"), out_o, 2e-2, "out")
    gu.check_close(lse.cpu().numpy(), lse_o, 2e-2, "lse")


def test_sinks_without_window_change_nothing():
    """With an unbounded left side the sink keys are already in the band:
    bit for bit the call without sinks."""
    base = dict(**RAGGED, num_q_heads=8, num_kv_heads=2, head_dim=128)
    gu.say("sinks without window")
    w0 = synth.custom(**base, name="nosink")
    w1 = synth.custom(**base, sink_keys=16, name="nosink")
    d = gu.to_device(w0)
    _, out0, lse0 = gu.run_hip(w0, d)
    d = gu.to_device(w1)
    _, out1, lse1 = gu.run_hip(w1, d)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert np.array_equal(lse0.cpu().numpy(), lse1.cpu().numpy())
