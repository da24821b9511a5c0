"""Benchmark: one step = the whole hot path (fused RoPE + KV append, then
ragged paged attention with its split-KV merge) over one batch of synthetic
input, inputs resident in HBM.

Headline (the JSON line's `value`): decode KV GB/s on the batched-decode
workload (32 sequences, KV lengths 512..4096, 32 query / 8 KV heads, D 128,
bf16, 16-token pages).  The same line carries the prefill TFLOP/s of the
ragged causal prefill workload (8192 tokens, bf16), the float8 long-context
decode and the sliding-window mixed batch, each with its dominant kernel's
roofline fraction, and the float64 oracle timed on the host as a CPU
baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only decode_bf16,...]
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR

Timing: W untimed warm-up steps, then K timed steps, the whole loop
bracketed by torch.cuda.synchronize().  Before every step a 1 GiB buffer is
read (outside the step's events) so that the 256 MB Infinity Cache and the
L2s hold none of the step's inputs -- a read, not a write, so that the step
does not pay for writing back someone else's dirty lines; each step is timed
with HIP events on the step's stream and ms_per_step is the median.  Kernel
durations come from the library's own events, attached to the kernels'
dispatches (nk_profile_*): inside the timed region only the workload's
dominant kernels carry them (a timestamped dispatch still costs the stream
about a microsecond); a second pass of the same number of steps times all
kernels for the per-kernel table.
"""

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
FLUSH_BYTES = 1 << 30
HIP_EVENT_NO_SYSTEM_FENCE = 0x20000000     # hipEventDisableSystemFence

METRIC = "decode KV GB/s (% HBM peak); prefill TFLOP/s (% bf16 MFMA peak)"
DESCR = {
    "decode_bf16": "batched decode, bf16: 32 seqs x 1 token, KV 512-4096, Hq32/Hkv8, D128, page16 permuted",
    "prefill_bf16": "ragged causal prefill, bf16: 8 segments 128..2176, 8192 tokens, Hq32/Hkv8, D128, page16",
    "decode_fp8": "long-context decode, e4m3 KV + f32 scales: 128 seqs, KV 4096-32768 log-uniform, Hq64/Hkv8, D128, split 512",
    "mixed_window_bf16": "sliding-window mixed batch, bf16: 4 prefill 1024-4096 + 60 decode 2048-8192, Hq16/Hkv8, D256, window 1024",
    "tiny_prefill_f32": "tiny ragged prefill, fp32: segments 5 and 12, Hq4/Hkv2, D64",
    "prefill_bidir_bf16": "the ragged prefill batch with every row seeing its whole segment (band unbounded on both sides)",
    "prefill_mrope_bf16": "the ragged prefill batch with M-RoPE: three position streams over 16/24/24 pairs",
    "prefill_prope_bf16": "the ragged prefill batch with p-RoPE: rotate-half pairs over the head, a quarter rotated",
    "mixed_sinks_bf16": "the sliding-window mixed batch with 4 sink keys beside the window (StreamingLLM)",
    "prefill_backward_bf16": "gradients (dq, dk, dv) of the ragged causal prefill batch from its forward's out and lse",
    "pack_bf16": "attention_pack of the decode batch's keys (32 slots with 64 spare rows each), Hkv8, D128, page16",
}
# kernels whose launches carry timing events inside the timed region
DOMINANT = {
    "decode_bf16": ("attn_decode",),
    "prefill_bf16": ("attn_prefill",),
    "decode_fp8": ("attn_decode",),
    "mixed_window_bf16": ("attn_prefill", "attn_decode"),
    "tiny_prefill_f32": ("attn_f32",),
    "prefill_bidir_bf16": ("attn_prefill",),
    "prefill_mrope_bf16": ("rope_write",),
    "prefill_prope_bf16": ("rope_write",),
    "mixed_sinks_bf16": ("attn_prefill", "attn_decode"),
}
KERNEL_SOURCES = ["attn_decode.hip", "attn_prefill.hip", "rope_write.hip", "lse_merge.hip", "common.h", "internal.h"]
# the sources a kernel family is built from: a counter summary stays valid
# while these are unchanged
FAMILY_SOURCES = {
    "attn_decode": ["attn_decode.hip", "common.h", "internal.h"],
    "attn_prefill": ["attn_prefill.hip", "common.h", "internal.h"],
    "rope_write": ["rope_write.hip", "common.h", "internal.h"],
    "pack_kernel": ["rope_write.hip", "common.h", "internal.h"],
    "_mfma_kernel": ["attn_backward.hip", "common.h", "internal.h"],
}
KERNEL_SOURCES = KERNEL_SOURCES + ["attn_backward.hip"]


def family_sources(kernel_name):
    for fam, files in FAMILY_SOURCES.items():
        if fam in kernel_name:
            return files
    return KERNEL_SOURCES


def source_hash(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "ragged_paged_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ GPU part
class Prepared:
    """One workload's inputs resident on the GPU."""


def prepare(name):
    import numpy as np
    import torch

    import synth
    from ragged_paged_kv_amd import nk

    w = synth.make(name)
    t0 = time.time()
    raw = synth.build_cache(w)
    nt = synth.new_tokens(w)
    dev = "cuda"

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    st = Prepared()
    st.w = w
    if w.in_dtype == "bf16":
        st.q, st.k, st.v = (t(nt[n].view(np.int16), torch.bfloat16) for n in ("q", "k", "v"))
    else:
        st.q, st.k, st.v = (t(nt[n]) for n in ("q", "k", "v"))
    if w.cache_dtype == "bf16":
        kp, vp = t(raw["k_pages"].view(np.int16), torch.bfloat16), t(raw["v_pages"].view(np.int16), torch.bfloat16)
    else:
        kp, vp = t(raw["k_pages"]), t(raw["v_pages"])
    ks = None if raw["k_scales"] is None else t(raw["k_scales"])
    vs = None if raw["v_scales"] is None else t(raw["v_scales"])
    del raw
    st.cache = nk.PagedKVCache(kp, vp, t(w.page_table.astype(np.int32)), ks, vs)
    st.q_offsets, st.kv_lens = t(w.q_offsets.astype(np.int32)), t(w.kv_lens.astype(np.int32))
    st.pos = None if w.position_ids is None else t(w.position_ids.astype(np.int32))
    if w.mrope_sections is not None:
        st.pos = t(synth.mrope_positions(w))
    st.freqs = t(synth.freqs_table(w))
    st.q_out = torch.empty_like(st.q)
    st.out = torch.empty_like(st.q)
    st.lse = torch.empty(w.total_q, w.num_q_heads, dtype=torch.float32, device=dev)
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s (cache {kp.numel() * kp.element_size() / 1e9:.2f} GB)")
    return st


class StepEvent:
    """A HIP event for timing only (no system-scope fence when recorded, so
    recording it neither writes back nor invalidates the caches), recorded
    on torch's current stream."""

    _hip = None

    def __init__(self):
        if StepEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            StepEvent._hip = hip
        self.ev = ctypes.c_void_p()
        rc = StepEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_NO_SYSTEM_FENCE)
        assert rc == 0, f"hipEventCreateWithFlags: {rc}"

    def record(self):
        import torch
        rc = StepEvent._hip.hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, f"hipEventRecord: {rc}"

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = StepEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        assert rc == 0, f"hipEventElapsedTime: {rc}"
        return ms.value

    def __del__(self):
        if self.ev:
            StepEvent._hip.hipEventDestroy(self.ev)


def measure(st, steps, warmup, flush, split=None):
    """Time `steps` hot-path steps on prepared inputs (see module doc)."""
    import torch

    from synth import work
    from ragged_paged_kv_amd import nk

    w = st.w
    split_req = w.split_tokens if split is None else split
    ws_bytes = nk.workspace_size(st.q.dtype, st.cache, w.num_seqs, w.total_q, w.max_q_len, w.max_kv_len,
                                 w.num_q_heads, w.window_left, split_req)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    split_used = nk.split_tokens(st.cache, w.num_seqs, w.max_kv_len, w.num_q_heads, w.window_left, split_req)
    min_q = int(w.q_lens.min())               # host bound: no decode launch for a prefill-only batch

    def step():
        nk.rope_qk_write_paged(st.q, st.k, st.v, st.q_offsets, st.kv_lens, st.freqs, st.cache, w.rotary_dim,
                               w.rope_layout, position_ids=st.pos, q_out=st.q_out, mrope_sections=w.mrope_sections)
        nk.ragged_paged_attention(st.q_out, st.q_offsets, st.kv_lens, st.cache, w.softmax_scale, w.max_q_len,
                                  w.max_kv_len, w.window_left, out=st.out, lse=st.lse, kv_split_tokens=split_req,
                                  workspace=ws, window_right=w.window_right,
                                  sink_keys=w.sink_keys, min_q_len=min_q)

    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def timed(nsteps, families):
        """nsteps steps, each after a cache-clearing read and between two
        events; the library brackets only the launches of `families`."""
        nk.profile_reset()
        if families:
            nk.profile_enable(True, families)
        evs = [(StepEvent(), StepEvent()) for _ in range(nsteps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for i in range(nsteps):
            if scratch is not None:
                torch.sum(scratch, dim=0, out=sink)
            evs[i][0].record()
            step()
            evs[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        nk.profile_enable(False)
        kern = {}
        for fam in nk.PROFILE_FAMILIES:
            tot, n = nk.profile_read(fam)
            if n:
                kern[fam] = {"avg_ms": tot / n, "launches": n}
        return sorted(a.elapsed_time(b) for a, b in evs), wall, kern

    # bring the GPU to its working clock first (it idles while the host
    # prepares inputs): ~0.2 s of the cache-clearing read, outside any step
    if scratch is not None:
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(20):
                torch.sum(scratch, dim=0, out=sink)
            torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: only the dominant kernels carry event pairs (each pair
    # costs the stream a few microseconds, which would otherwise show up in
    # the step time); a second pass of the same steps times every kernel
    times, wall, kern_timed = timed(steps, DOMINANT[w.name])
    ms = times[len(times) // 2]
    _, _, kern = timed(steps, nk.PROFILE_FAMILIES)
    for fam, rec in kern_timed.items():
        kern[fam] = rec
    res = {
        "workload": w.name, "descr": DESCR[w.name], "ms_per_step": ms, "ms_min": times[0], "ms_max": times[-1],
        "wall_s_incl_flush": wall, "kernels": kern, "kernels_timed_in_region": sorted(kern_timed),
        "split_tokens": split_used,
        "decode_bytes": work.decode_bytes(w), "prefill_flops": work.prefill_flops(w), "rope_bytes": work.rope_bytes(w),
    }
    if res["decode_bytes"]:
        res["decode_GBps_step"] = res["decode_bytes"] / ms / 1e6
        if "attn_decode" in kern:
            res["decode_GBps_kernel"] = res["decode_bytes"] / kern["attn_decode"]["avg_ms"] / 1e6
    if res["prefill_flops"]:
        res["prefill_TFLOPs_step"] = res["prefill_flops"] / ms / 1e9
        if "attn_prefill" in kern:
            res["prefill_TFLOPs_kernel"] = res["prefill_flops"] / kern["attn_prefill"]["avg_ms"] / 1e9
    if "rope_write" in kern:
        res["rope_GBps_kernel"] = res["rope_bytes"] / kern["rope_write"]["avg_ms"] / 1e6
    del scratch, ws
    return res


def measure_pack(steps, warmup, flush):
    """nk_attention_pack of the decode batch's keys: 32 slots of kv_len + 64
    rows each (spare room, left out through key_lengths), Hkv 8, D 128,
    bf16 rows into 16-token pages.  Algorithmic bytes: the kept K and V rows
    read once and written once, plus the offsets, lengths and table."""
    import numpy as np
    import torch

    import synth

    from ragged_paged_kv_amd import nk

    w = synth.make("decode_bf16")
    kept = w.kv_lens.astype(np.int64)
    slots = kept + 64
    offs = np.concatenate([[0], np.cumsum(slots)]).astype(np.int32)
    rows, hkv, d, P = int(offs[-1]), w.num_kv_heads, w.head_dim, 16
    gen = torch.Generator(device="cuda").manual_seed(7)
    k = torch.randn(rows, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(rows, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    d_offs = torch.from_numpy(offs).cuda()
    d_lens = torch.from_numpy(kept.astype(np.int32)).cuda()
    cache, kv_lens, max_len = nk.attention_pack(k, v, d_offs, d_lens, page_size=P, max_key_len=int(kept.max()))
    c = cache.struct()
    B = len(kept)

    def step():
        st = nk.lib().nk_attention_pack(k.data_ptr(), v.data_ptr(), nk.NK_BF16, d_offs.data_ptr(),
                                        d_lens.data_ptr(), ctypes.byref(c), kv_lens.data_ptr(), B, max_len,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == nk.NK_OK

    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    nk.profile_reset()
    nk.profile_enable(True, ["attention_pack"])
    evs = [(StepEvent(), StepEvent()) for _ in range(steps)]
    for i in range(steps):
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    nk.profile_enable(False)
    times = sorted(a.elapsed_time(b) for a, b in evs)
    tot, n = nk.profile_read("attention_pack")
    kb = int(kept.sum()) * hkv * d * 2 * 2
    nbytes = 2 * kb + (B + 1) * 4 + B * 4 + int(((kept + P - 1) // P).sum()) * 4 + B * 4
    ms = times[len(times) // 2]
    res = {"workload": "pack_bf16", "descr": DESCR["pack_bf16"], "ms_per_step": ms, "ms_min": times[0],
           "ms_max": times[-1], "kernels": {"attention_pack": {"avg_ms": tot / n, "launches": n}},
           "kernels_timed_in_region": ["attention_pack"], "pack_bytes": nbytes,
           "pack_GBps_kernel": nbytes / (tot / n) / 1e6}
    del scratch
    return res


def measure_backward(steps, warmup, flush):
    """nk_ragged_paged_attention_backward on the ragged prefill batch: its
    forward (RoPE + append + attention) once, a seeded output gradient, then
    the timed gradient calls.  Algorithmic flops: 10 D per (row, head, visible
    key) -- the score recomputation, dO V^T, dV, dQ and dK products."""
    import numpy as np
    import torch

    from ragged_paged_kv_amd import nk
    from synth import work

    st = prepare("prefill_bf16")
    w = st.w
    nk.rope_qk_write_paged(st.q, st.k, st.v, st.q_offsets, st.kv_lens, st.freqs, st.cache, w.rotary_dim,
                           w.rope_layout, position_ids=st.pos, q_out=st.q_out)
    nk.ragged_paged_attention(st.q_out, st.q_offsets, st.kv_lens, st.cache, w.softmax_scale, w.max_q_len,
                              w.max_kv_len, w.window_left, out=st.out, lse=st.lse)
    gen = torch.Generator(device="cuda").manual_seed(5)
    dout = torch.randn(st.q.shape, generator=gen, device="cuda").to(torch.bfloat16)
    key_offsets = np.concatenate([[0], np.cumsum(w.kv_lens)]).astype(np.int32)
    d_koffs = torch.from_numpy(key_offsets).cuda()
    rows = int(key_offsets[-1])
    dq = torch.empty(w.total_q, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    dk = torch.empty(rows, w.num_kv_heads, w.head_dim, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)

    def step():
        nk.ragged_paged_attention_backward(st.q_out, st.q_offsets, st.kv_lens, st.cache, w.softmax_scale,
                                           w.max_kv_len, st.out, dout, st.lse, d_koffs, rows, w.window_left,
                                           dq=dq, dk=dk, dv=dv)

    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if flush else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    nk.profile_reset()
    nk.profile_enable(True, ["attn_backward"])
    evs = [(StepEvent(), StepEvent()) for _ in range(steps)]
    for i in range(steps):
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)
        evs[i][0].record()
        step()
        evs[i][1].record()
    torch.cuda.synchronize()
    nk.profile_enable(False)
    times = sorted(a.elapsed_time(b) for a, b in evs)
    tot, n = nk.profile_read("attn_backward")
    flops = 10 * w.head_dim * w.num_q_heads * work.prefill_pairs(w)
    ms = times[len(times) // 2]
    res = {"workload": "prefill_backward_bf16", "descr": DESCR["prefill_backward_bf16"], "ms_per_step": ms,
           "ms_min": times[0], "ms_max": times[-1],
           "kernels": {"attn_backward": {"avg_ms": tot / n, "launches": n}},
           "kernels_timed_in_region": ["attn_backward"], "backward_flops": flops,
           "backward_TFLOPs_kernel": flops / (tot / n) / 1e9}
    del scratch, st
    return res


def run_workload(name, steps, warmup, flush):
    import torch
    if name == "prefill_backward_bf16":
        res = measure_backward(steps, warmup, flush)
        torch.cuda.empty_cache()
        return res
    if name == "pack_bf16":
        res = measure_pack(steps, warmup, flush)
        torch.cuda.empty_cache()
        return res
    st = prepare(name)
    res = measure(st, steps, warmup, flush)
    del st
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU baseline
CPU_BASELINE_SECONDS = 12.0     # host time budget of the headline workload's oracle sample
CPU_WORKLOAD_SECONDS = 4.0      # the same for every other workload
CPU_MAX_WORKERS = 16            # host cores a GPU's share of the machine holds

_ORACLE_WORKLOADS = {}
# workloads whose oracle task is not the forward pass of their own batch
_ORACLE_SOURCE = {"pack_bf16": "decode_bf16", "prefill_backward_bf16": "prefill_bf16"}


def _oracle_inputs(w):
    """Rotated queries and the cache after the append, by the oracle (the
    forward's inputs; not timed)."""
    import numpy as np

    import synth
    from oracle import formats

    raw = synth.build_cache(w, threads=1)
    nt = synth.new_tokens(w)
    conv = (lambda x: x.astype(np.float64)) if w.in_dtype == "f32" else formats.bf16_value
    q, k, v = conv(nt["q"]), conv(nt["k"]), conv(nt["v"])
    return raw, q, k, v


def _oracle_segment(name, s, r0, r1):
    """Rows r0..r1-1 of segment s of a workload through the oracle, in a
    worker process with one BLAS thread; returns the kind of work, its
    algorithmic amount and the oracle's seconds.  Inputs are generated before
    the clock starts.  A block of a segment's rows is run as a segment of its
    own over the keys those rows can reach (the prefix up to the block's last
    position), so its rows sit at their original positions; values other
    than the block's own tokens come from the segment's prior-row stream
    (the same shapes and work, other numbers).
      forward workloads: RoPE + append, then attention (decode bytes or
        prefill flops of the segment);
      pack_bf16: slot s of the pack (kv_len kept rows of kv_len + 64), bytes;
      prefill_backward_bf16: the gradients of segment s, 10 D flops per
        (row, head, visible key)."""
    from dataclasses import replace

    import numpy as np
    import threadpoolctl

    import synth
    from oracle import attention as o_attn
    from oracle import pack as o_pack
    from oracle import rope as o_rope
    from oracle.paged import PagedCache
    from synth import work

    src = _ORACLE_SOURCE.get(name, name)
    if src not in _ORACLE_WORKLOADS:
        _ORACLE_WORKLOADS[src] = synth.make(src)
    w = _ORACLE_WORKLOADS[src].subset([s])
    q_len, kv_len = int(w.q_lens[0]), int(w.kv_lens[0])
    if (r0, r1) != (0, q_len):
        w = replace(w, q_lens=np.array([r1 - r0], np.int32), kv_lens=np.array([kv_len - q_len + r1], np.int32),
                    token_ids=w.token_ids[r0:r1].copy())
    with threadpoolctl.threadpool_limits(1):
        if name == "pack_bf16":
            kept = int(w.kv_lens[0])
            rng = np.random.default_rng(s)
            k = rng.standard_normal((kept + 64, w.num_kv_heads, w.head_dim))
            v = rng.standard_normal((kept + 64, w.num_kv_heads, w.head_dim))
            t0 = time.perf_counter()
            o_pack.attention_pack(k, v, np.array([0, kept + 64]), np.array([kept]), "bf16", 16)
            dt = time.perf_counter() - t0
            nbytes = 2 * kept * w.num_kv_heads * w.head_dim * 2 * 2 + 16 + (-(-kept // 16)) * 4
            return "pack", nbytes, dt
        raw, q, k, v = _oracle_inputs(w)
        freqs = synth.freqs_table(w)
        t0 = time.perf_counter()
        cache = PagedCache.from_storage(w.cache_dtype, raw["k_pages"], raw["v_pages"], raw["k_scales"],
                                        raw["v_scales"])
        q_out, cache2 = o_rope.rope_qk_write_paged(q, k, v, w.in_dtype, w.q_offsets, w.kv_lens, w.position_ids,
                                                   freqs, w.rotary_dim, w.rope_layout, cache, w.page_table)
        if name == "prefill_backward_bf16":
            dout = np.random.default_rng(s).standard_normal(q_out.shape)
            t0 = time.perf_counter()
            o_attn.ragged_paged_attention_backward(q_out, w.q_offsets, w.kv_lens, cache2, w.page_table,
                                                   w.softmax_scale, dout, w.window_left,
                                                   window_right=w.window_right, sink_keys=w.sink_keys)
            dt = time.perf_counter() - t0
            return "backward", 10 * w.head_dim * w.num_q_heads * work.prefill_pairs(w), dt
        o_attn.ragged_paged_attention(q_out, w.q_offsets, w.kv_lens, cache2, w.page_table, w.softmax_scale,
                                      w.window_left, window_right=w.window_right, sink_keys=w.sink_keys)
        dt = time.perf_counter() - t0
    if int(w.q_lens[0]) == 1:
        return "decode", work.decode_bytes(w), dt
    return "prefill", work.prefill_flops(w), dt


_KIND_UNIT = {"decode": ("GB/s", 1e9), "prefill": ("TFLOP/s", 1e12), "pack": ("GB/s", 1e9),
              "backward": ("TFLOP/s", 1e12)}


def cpu_baseline(name, seconds, pool, cores):
    """The oracle as it stands, on the host's cores: a pool of `cores`
    processes, one BLAS thread each, takes the workload's segments one at a
    time (blocks of at most 256 rows, 64 for the gradients; a seeded
    shuffle of their order, at most four passes) until
    `seconds` of wall time have passed, then lets the segments in flight
    finish.  The rate of each kind of work is its amount over its oracle
    seconds summed over the segment runs, times the number of processes:
    the processes run side by side, so that is the pool's aggregate rate.
    Returns {kind: {value, unit, cores, kind, sample}}."""
    import concurrent.futures as cf

    import numpy as np

    import synth

    w = synth.make(_ORACLE_SOURCE.get(name, name))
    n_seg = w.num_seqs
    block = 64 if name == "prefill_backward_bf16" else 256
    tasks = [(s, r0, min(r0 + block, int(w.q_lens[s]))) for s in range(n_seg)
             for r0 in range(0, max(int(w.q_lens[s]), 1), block)]
    order = np.random.default_rng(1234).permutation(len(tasks))
    done = {}
    t0 = time.perf_counter()
    pending, i = set(), 0
    while True:
        while len(pending) < cores and time.perf_counter() - t0 < seconds and i < 4 * len(tasks):
            pending.add(pool.submit(_oracle_segment, name, *tasks[order[i % len(tasks)]]))
            i += 1
        if not pending:
            break
        fin, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
        for f in fin:
            kind, amount, dt = f.result()
            rec = done.setdefault(kind, [0, 0.0, 0])
            rec[0] += amount
            rec[1] += dt
            rec[2] += 1
    wall = time.perf_counter() - t0
    res = {}
    for kind, (amount, secs, n) in done.items():
        unit, scale = _KIND_UNIT[kind]
        res[kind] = {"value": amount / secs * cores / scale, "unit": unit, "cores": cores, "kind": "oracle",
                     "sample": f"{n} runs of row blocks ({kind} work; {len(tasks)} blocks in {n_seg} segments), "
                               f"{cores} processes x 1 BLAS thread, {wall:.1f} s wall; oracle {secs:.1f} s summed "
                               f"over the runs"}
    return res


def cpu_cores():
    """Host cores this process may run on, capped at one GPU's share."""
    return max(1, min(len(os.sched_getaffinity(0)), CPU_MAX_WORKERS))


# ------------------------------------------------------------------ counters
# the counter summary (profiles/traffic_KEY.json) of each workload's HBM-bound kernel
TRAFFIC_KEYS = {"decode_bf16": "decode_bf16", "decode_fp8": "decode_fp8", "mixed_window_bf16": "decode_d256",
                "prefill_bf16": "rope_prefill", "pack_bf16": "pack"}


def load_traffic(kernel_key):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(family_sources(rec.get("kernel", ""))):
        return None
    return rec.get("bytes_per_launch")


def load_mfma(workload):
    """MFMA counter summary of a workload's prefill kernel from profiles/,
    if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(family_sources(rec.get("kernel", ""))):
        return None
    return {k: rec.get(k) for k in ("executed_over_algorithmic", "mfma_busy_frac")}


def _short(name):
    """Kernel name without namespaces / argument lists, template arguments kept."""
    n = name.replace("nk::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0] if "(" in n else n


def rocpd_summary(db_path, title, command):
    """Per-kernel dispatch statistics of a rocprofv3 --kernel-trace database
    (rocpd SQLite), grouped by kernel and grid; returns the text table."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, grid_x, grid_y, grid_z, workgroup_x, vgpr_count, accum_vgpr_count, "
                       "lds_size, scratch_size, duration from kernels").fetchall()
    groups = {}
    for name, gx, gy, gz, wx, vg, ag, lds, scr, dur in rows:
        key = (_short(name), gx, gy, gz, wx, vg, ag, lds, scr)
        groups.setdefault(key, []).append(dur / 1000.0)
    lines = [f"# {title}", f"# command: {command}", "#",
             "# kernel | grid (threads x,y,z) | block | vgpr+agpr | lds B | scratch B | calls | avg us | min us | max us"]
    for key, ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        n, gx, gy, gz, wx, vg, ag, lds, scr = key
        lines.append(f"{n} | {gx},{gy},{gz} | {wx} | {vg}+{ag} | {lds} | {scr} | {len(ds)} | "
                     f"{sum(ds) / len(ds):.2f} | {min(ds):.2f} | {max(ds):.2f}")
    return "\n".join(lines) + "\n"


def rocpd_counter(db_path, kernel_match, counter):
    """Average value of a counter over the dispatches of matching kernels."""
    import sqlite3
    con = sqlite3.connect(db_path)
    vals = [v for name, cn, v in con.execute("select kernel_name, counter_name, value from counters_collection")
            if kernel_match in name and cn == counter]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def rocpd_mfma(db_path, kernel_match, simds, gui_instances, flops_per_launch):
    """MFMA work and utilisation of the matching kernel from one rocprofv3
    --pmc pass over MFMA_COUNTERS: bf16 MFMA flops executed per dispatch
    (512 per MOPS unit), and the busy cycles of the matrix units over the
    dispatch's active GPU cycles times the SIMD count (GRBM_GUI_ACTIVE is read
    once per XCD, hence `gui_instances`)."""
    vals = {c: rocpd_counter(db_path, kernel_match, c) for c in MFMA_COUNTERS}
    mops, n = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    busy, _ = vals["SQ_VALU_MFMA_BUSY_CYCLES"]
    gui, _ = vals["GRBM_GUI_ACTIVE"]
    rec = {"kernel": kernel_match, "dispatches": n, "counters_per_dispatch": {c: v[0] for c, v in vals.items()},
           "simds": simds, "gui_instances": gui_instances, "algorithmic_flops_per_launch": flops_per_launch}
    if mops is not None:
        rec["mfma_flops_per_dispatch"] = 512.0 * mops
        if flops_per_launch:
            rec["executed_over_algorithmic"] = 512.0 * mops / flops_per_launch
    if busy is not None and gui:
        rec["active_cycles"] = gui / gui_instances
        rec["mfma_busy_frac"] = busy / (gui / gui_instances * simds)
    rec["source_hash"] = source_hash(family_sources(kernel_match))
    return rec


def _pmc_rows(d):
    import csv
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, kernel_match, key):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the kernel, scaled
    by the same counters on a plain copy of known size; writes
    profiles/traffic_<key>.json and prints the summary."""
    def avg(rows, match, counter):
        vals = [float(r.get("Counter_Value", r.get("counter_value", 0))) for r in rows
                if match in r.get("Kernel_Name", r.get("kernel_name", "")) and
                r.get("Counter_Name", r.get("counter_name", "")) == counter]
        return sum(vals) / len(vals) if vals else None
    kf = avg(_pmc_rows(fetch_dir), kernel_match, "FETCH_SIZE")
    kw = avg(_pmc_rows(write_dir), kernel_match, "WRITE_SIZE")
    cf = avg(_pmc_rows(copy_fetch_dir), "copy", "FETCH_SIZE") or avg(_pmc_rows(copy_fetch_dir), "elementwise", "FETCH_SIZE")
    cw = avg(_pmc_rows(copy_write_dir), "copy", "WRITE_SIZE") or avg(_pmc_rows(copy_write_dir), "elementwise", "WRITE_SIZE")
    fs = copy_bytes / (cf * 1024.0) if cf else None
    wsf = copy_bytes / (cw * 1024.0) if cw else None
    rec = {"kernel": kernel_match, "fetch_kib": kf, "write_kib": kw, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "copy_bytes": copy_bytes, "fetch_scale": fs, "write_scale": wsf,
           "bytes_per_launch": (kf * 1024 * fs + kw * 1024 * wsf) if None not in (kf, kw, fs, wsf) else None,
           "source_hash": source_hash(family_sources(kernel_match))}
    with open(os.path.join(ROOT, "profiles", f"traffic_{key}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="decode_bf16,prefill_bf16,decode_fp8,mixed_window_bf16,prefill_bidir_bf16,"
                    "mixed_sinks_bf16,prefill_mrope_bf16,prefill_prope_bf16,pack_bf16,prefill_backward_bf16")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    ap.add_argument("--pmc-kernel", default="attn_decode_kernel")
    ap.add_argument("--pmc-key", default="decode_bf16")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--copy-only", action="store_true", help="run one plain 1 GiB copy (counter calibration)")
    ap.add_argument("--rocpd-summary", nargs=3, metavar=("DB", "OUT", "COMMAND"),
                    help="write the per-kernel table of a rocprofv3 kernel-trace database")
    ap.add_argument("--rocpd-mfma", nargs=2, metavar=("DB", "OUT"),
                    help="MFMA flops and busy fraction of --pmc-kernel from a pass over MFMA_COUNTERS")
    ap.add_argument("--mfma-workload", default="prefill_bf16",
                    help="workload whose algorithmic prefill flops --rocpd-mfma compares with")
    ap.add_argument("--simds", type=int, default=1024, help="SIMDs of the GPU (MI355X: 256 CUs x 4)")
    ap.add_argument("--gui-instances", type=int, default=8, help="GRBM_GUI_ACTIVE readings summed per dispatch (XCDs)")
    ap.add_argument("--rocpd-traffic", nargs=5, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB", "OUT"),
                    help="HBM bytes per launch of --pmc-kernel from FETCH_SIZE / WRITE_SIZE databases")
    args = ap.parse_args()

    if args.rocpd_summary:
        db, out, cmd = args.rocpd_summary
        text = rocpd_summary(db, "rocprofv3 --kernel-trace --stats: per-kernel dispatch durations", cmd)
        with open(out, "w") as f:
            f.write(text)
        print(text)
        return 0
    if args.rocpd_mfma:
        import synth
        from synth import work
        db, out = args.rocpd_mfma
        if args.mfma_workload == "prefill_backward_bf16":
            # gradients: 10 D per visible (row, head, key) against the forward's 4 D
            flops = work.prefill_flops(synth.make("prefill_bf16")) * 10 // 4
        else:
            flops = work.prefill_flops(synth.make(args.mfma_workload))
        rec = rocpd_mfma(db, args.pmc_kernel, args.simds, args.gui_instances, flops)
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return 0
    if args.rocpd_traffic:
        fdb, wdb, cfdb, cwdb, out = args.rocpd_traffic
        kf, nf = rocpd_counter(fdb, args.pmc_kernel, "FETCH_SIZE")
        kw, nw = rocpd_counter(wdb, args.pmc_kernel, "WRITE_SIZE")
        cf, _ = rocpd_counter(cfdb, "copyBuffer", "FETCH_SIZE")
        cw, _ = rocpd_counter(cwdb, "copyBuffer", "WRITE_SIZE")
        if cf is None:
            cf, _ = rocpd_counter(cfdb, "elementwise", "FETCH_SIZE")
            cw, _ = rocpd_counter(cwdb, "elementwise", "WRITE_SIZE")
        fs = args.copy_bytes / (cf * 1024.0) if cf else None
        wsf = args.copy_bytes / (cw * 1024.0) if cw else None
        rec = {"kernel": args.pmc_kernel, "dispatches": [nf, nw], "fetch_kib_per_dispatch": kf,
               "write_kib_per_dispatch": kw, "copy_bytes": args.copy_bytes, "copy_fetch_kib": cf,
               "copy_write_kib": cw, "fetch_scale": fs, "write_scale": wsf,
               "bytes_per_launch": (kf * 1024 * fs + kw * 1024 * wsf) if None not in (kf, kw, fs, wsf) else None,
               "source_hash": source_hash(family_sources(args.pmc_kernel))}
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return 0

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.copy_bytes, args.pmc_kernel, args.pmc_key)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each GPU would run the same kernels on its own share of sequences or KV heads).",
              file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "no GPU"
    if args.copy_only:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        return 0

    names = [n for n in args.only.split(",") if n]
    results = {}
    for n in names:
        log(f"running {n}")
        results[n] = run_workload(n, args.steps, args.warmup, not args.no_flush)
        log(json.dumps(results[n]))

    head = results.get("decode_bf16") or next(iter(results.values()))
    cpu, cpu_all = None, {}
    if not args.no_cpu:
        import concurrent.futures as cf
        import multiprocessing as mp
        cores = cpu_cores()
        log(f"timing the oracle on the host ({cores} processes)")
        with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as pool:
            for n in names:
                budget = CPU_BASELINE_SECONDS if n == head["workload"] else CPU_WORKLOAD_SECONDS
                cpu_all[n] = cpu_baseline(n, budget, pool, cores)
                log(n, json.dumps(cpu_all[n]))
        hk = cpu_all.get(head["workload"], {})
        cpu = hk.get("decode") or next(iter(hk.values()), None)

    dec_k = head.get("kernels", {}).get("attn_decode")
    roof = None
    if dec_k:
        achieved = head["decode_bytes"] / dec_k["avg_ms"] / 1e6
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic("decode_bf16"),
                "kernel": "attn_decode_kernel<128,16,bf16>", "avg_kernel_ms": dec_k["avg_ms"],
                "bytes_per_launch": head["decode_bytes"]}
    value = head.get("decode_GBps_step", 0.0)
    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head["workload"] + ": " + head["descr"], "global_batch": 32, "seq_len": "512-4096 KV",
                   "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    extra = {}
    for n, r in results.items():
        e = {"ms_per_step": r["ms_per_step"], "kernels": r["kernels"], "split_tokens": r.get("split_tokens")}
        if r.get("backward_TFLOPs_kernel"):
            e["backward_TFLOPs_kernel"] = r["backward_TFLOPs_kernel"]
            e["backward_mfma_frac"] = r["backward_TFLOPs_kernel"] / BF16_PEAK_TFLOPS
        if r.get("pack_GBps_kernel"):
            e["pack_GBps_kernel"] = r["pack_GBps_kernel"]
            e["pack_hbm_frac"] = r["pack_GBps_kernel"] / HBM_PEAK_GBS
        if r.get("decode_GBps_kernel"):
            e["decode_GBps_kernel"] = r["decode_GBps_kernel"]
            e["decode_hbm_frac"] = r["decode_GBps_kernel"] / HBM_PEAK_GBS
        if r.get("prefill_TFLOPs_kernel"):
            e["prefill_TFLOPs_kernel"] = r["prefill_TFLOPs_kernel"]
            e["prefill_mfma_frac"] = r["prefill_TFLOPs_kernel"] / BF16_PEAK_TFLOPS
            e["prefill_mfma_counters"] = load_mfma(n)
        if r.get("rope_GBps_kernel"):
            e["rope_GBps_kernel"] = r["rope_GBps_kernel"]
        if r.get("decode_bytes") and r.get("prefill_flops"):
            # one ragged call, two launches: the time each would take at its
            # roofline over the time the attention kernels took together
            ks = r["kernels"]
            t_attn = sum(ks[f]["avg_ms"] for f in ("attn_decode", "attn_prefill", "lse_merge") if f in ks) / 1e3
            if t_attn > 0:
                ideal = r["decode_bytes"] / (HBM_PEAK_GBS * 1e9) + r["prefill_flops"] / (BF16_PEAK_TFLOPS * 1e12)
                e["combined_roofline_frac"] = ideal / t_attn
        key = TRAFFIC_KEYS.get(n)
        traffic = load_traffic(key) if key else None
        if traffic:
            # HBM bytes per launch of the workload's HBM-bound kernel, from the
            # committed counter summary, over its algorithmic bytes
            alg = {"decode_bf16": r.get("decode_bytes"), "decode_fp8": r.get("decode_bytes"),
                   "mixed_window_bf16": r.get("decode_bytes"), "prefill_bf16": r.get("rope_bytes"),
                   "pack_bf16": r.get("pack_bytes")}.get(n)
            e["traffic"] = {"kernel_key": key, "bytes_per_launch": traffic,
                            "over_algorithmic": traffic / alg if alg else None}
        if n in cpu_all:
            e["cpu_baseline"] = cpu_all[n]
        extra[n] = e
    line["workloads"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
