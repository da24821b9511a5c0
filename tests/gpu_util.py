"""Helpers of the GPU parity tests: put a synthetic workload on the GPU, run
the HIP path through the C ABI, run the oracle on the same inputs, compare.

Tolerances (on out and lse, against the oracle's float64 values computed from
the same stored inputs): 1e-4 for float32 inputs, 2e-2 for bf16 inputs,
6e-2 with an e4m3 cache.  Stored intermediates (q_out, appended cache rows,
e4m3 codes and scales) must be bit-equal to the oracle's: both sides round
the float64 rotation once to the storage format.
"""

import sys
import time

import numpy as np
import torch

import synth
from oracle import attention as o_attn
from oracle import formats, rope as o_rope
from oracle.paged import PagedCache
from ragged_paged_kv_amd import nk

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2}


# (case, max |out error|, max |lse error|, tolerance) of the compared runs,
# printed in the test run's terminal summary
MARGINS = []


def record_margin(case, err_out, err_lse, tol):
    MARGINS.append((case, float(err_out), float(err_lse), float(tol)))


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def tol_for(w):
    if w.cache_dtype == "e4m3":
        return TOL["e4m3"]
    return TOL[w.in_dtype]


def _t(x, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev)


def to_device(w, dev="cuda", cache=None):
    """Device tensors of a workload: new tokens, offsets, table, cache."""
    nt = synth.new_tokens(w)
    tdt = torch.float32 if w.in_dtype == "f32" else torch.bfloat16
    store = (lambda a: _t(a, dev)) if w.in_dtype == "f32" else (lambda a: _t(a.view(np.int16), dev, torch.bfloat16))
    raw = synth.build_cache(w) if cache is None else cache
    if w.cache_dtype == "f32":
        kp, vp = _t(raw["k_pages"], dev), _t(raw["v_pages"], dev)
    elif w.cache_dtype == "bf16":
        kp = _t(raw["k_pages"].view(np.int16), dev, torch.bfloat16)
        vp = _t(raw["v_pages"].view(np.int16), dev, torch.bfloat16)
    else:
        kp, vp = _t(raw["k_pages"], dev), _t(raw["v_pages"], dev)
    ks = None if raw["k_scales"] is None else _t(raw["k_scales"], dev)
    vs = None if raw["v_scales"] is None else _t(raw["v_scales"], dev)
    d = dict(q=store(nt["q"]), k=store(nt["k"]), v=store(nt["v"]),
             q_offsets=_t(w.q_offsets.astype(np.int32), dev), kv_lens=_t(w.kv_lens.astype(np.int32), dev),
             position_ids=None if w.position_ids is None else _t(w.position_ids.astype(np.int32), dev),
             freqs=_t(synth.freqs_table(w), dev), raw_cache=raw, tokens=nt, dtype=tdt)
    d["cache"] = nk.PagedKVCache(kp, vp, _t(w.page_table.astype(np.int32), dev), ks, vs)
    return d


def run_hip(w, d, split=None, out_lse=True):
    """RoPE + append, then attention, on the current stream."""
    q_out = nk.rope_qk_write_paged(d["q"], d["k"], d["v"], d["q_offsets"], d["kv_lens"], d["freqs"],
                                   d["cache"], w.rotary_dim, w.rope_layout, position_ids=d["position_ids"])
    lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device=q_out.device) if out_lse else None
    out, lse = nk.ragged_paged_attention(q_out, d["q_offsets"], d["kv_lens"], d["cache"], w.softmax_scale,
                                         w.max_q_len, w.max_kv_len, w.window_left, lse=lse,
                                         window_right=w.window_right, sink_keys=w.sink_keys,
                                         kv_split_tokens=w.split_tokens if split is None else split,
                                         min_q_len=int(w.q_lens.min()) if w.num_seqs else 0)
    return q_out, out, lse


def host_values(t, dtype):
    """Device tensor -> float64 numpy values of the stored elements."""
    t = t.detach().cpu()
    if dtype == "f32":
        return t.numpy().astype(np.float64)
    if dtype == "bf16":
        return formats.bf16_value(t.view(torch.int16).numpy().view(np.uint16))
    return formats.e4m3_value(t.view(torch.uint8).numpy())


def oracle_run(w, raw_cache=None):
    """The oracle on a workload (or a subset): returns q_out, cache, out, lse."""
    nt = synth.new_tokens(w)
    conv = (lambda a: a.astype(np.float64)) if w.in_dtype == "f32" else formats.bf16_value
    q, k, v = conv(nt["q"]), conv(nt["k"]), conv(nt["v"])
    raw = synth.build_cache(w) if raw_cache is None else raw_cache
    cache = PagedCache.from_storage(w.cache_dtype, raw["k_pages"], raw["v_pages"], raw["k_scales"], raw["v_scales"])
    q_out, cache2 = o_rope.rope_qk_write_paged(q, k, v, w.in_dtype, w.q_offsets, w.kv_lens, w.position_ids,
                                               synth.freqs_table(w), w.rotary_dim, w.rope_layout, cache,
                                               w.page_table)
    out, lse = o_attn.ragged_paged_attention(q_out, w.q_offsets, w.kv_lens, cache2, w.page_table,
                                             w.softmax_scale, w.window_left, window_right=w.window_right,
                                             sink_keys=w.sink_keys)
    return q_out, cache2, out, lse


def ulp_distance_bf16(a, b):
    """Distance in bf16 steps between two arrays of bf16 values."""
    ia = formats.bf16_bits(a).astype(np.int32)
    ib = formats.bf16_bits(b).astype(np.int32)
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia & 0x8000, 0x8000 - ia, ia)
    ib = np.where(ib & 0x8000, 0x8000 - ib, ib)
    return np.abs(ia - ib)


def compare_storage(gpu_vals, ref_vals, dtype, what):
    """Stored values (q_out, appended cache rows): bit-equal to the oracle's
    rounding of its float64 result.  Returns 0.0 (the differing fraction)."""
    g = np.asarray(gpu_vals, dtype=np.float64)
    r = np.asarray(ref_vals, dtype=np.float64)
    same = (g == r) | (np.isnan(g) & np.isnan(r))
    if not np.all(same):
        idx = np.unravel_index(int(np.argmin(same)), same.shape)
        n_bad = int(np.sum(~same))
        if dtype == "bf16":
            dist = ulp_distance_bf16(g, r)
            raise AssertionError(f"{what}: {n_bad} stored values differ (max {dist.max()} bf16 steps), "
                                 f"first at {tuple(int(i) for i in idx)}: gpu {g[idx]!r} oracle {r[idx]!r}")
        raise AssertionError(f"{what}: {n_bad} stored values differ, first at {tuple(int(i) for i in idx)}: "
                             f"gpu {g[idx]!r} oracle {r[idx]!r}")
    return 0.0


def check_close(gpu, ref, tol, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    assert not np.any(np.isnan(err)), f"{what}: NaN in result"
    m = float(err.max()) if err.size else 0.0
    if m > tol:
        idx = np.unravel_index(int(np.argmax(err)), err.shape)
        n_bad = int(np.sum(err > tol))
        raise AssertionError(f"{what}: max abs error {m:.3g} > {tol} at {tuple(int(i) for i in idx)} "
                             f"(gpu {gpu[idx]:.6g}, oracle {ref[idx]:.6g}); {n_bad} elements over")
    return m


class Timer:
    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        self.dt = time.time() - self.t
