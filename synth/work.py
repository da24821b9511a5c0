"""Algorithmic work of a workload: the bytes and flops the method must move
or compute (not the dense work a kernel may also spend).

* Decode bytes per sequence with n visible keys (n = min(kv_len, window)):
  ``n*Hkv*D*2*e_kv`` (K and V) ``+ [fp8] n*Hkv*2*4`` (scales)
  ``+ Hq*D*(e_q + e_out)`` (query in, output out) ``+ ceil(n/P)*4`` (page
  table) ``+ Hq*4`` (log-sum-exp).  The K+V term is the per-layer form of the
  Algenta page's ``kv_cache_memory_bytes`` (2 x layers x heads x d_head x
  seq_len x batch x bytes per element).
* Prefill flops: ``4 * D * Hq * sum over query rows of visible keys`` (2 for
  Q.K^T, 2 for P.V); masked halves of diagonal tiles are not credited.
* RoPE + append bytes: q in/out, k and v in, cache rows out (+ scales), the
  table rows read.
"""

import numpy as np

ELEM = {"f32": 4, "bf16": 2, "e4m3": 1}


def visible_keys(w):
    """Visible-key count of every query row (int64 [T])."""
    offs = w.q_offsets
    out = np.empty(w.total_q, dtype=np.int64)
    for s in range(w.num_seqs):
        ql, L = int(w.q_lens[s]), int(w.kv_lens[s])
        p = np.arange(ql) + L - ql
        hi = np.full_like(p, L - 1) if w.window_right < 0 else np.minimum(p + w.window_right, L - 1)
        lo = np.zeros_like(p) if w.window_left < 0 else np.maximum(0, p - w.window_left)
        sinks = np.maximum(0, np.minimum(np.minimum(lo, hi + 1), w.sink_keys if w.window_left >= 0 else 0))
        out[offs[s]:offs[s] + ql] = np.maximum(hi - lo + 1, 0) + sinks
    return out


def is_decode(w, max_decode_q=1):
    return (w.q_lens <= max_decode_q) & (w.q_lens > 0)


def decode_bytes(w, seqs=None):
    """Algorithmic bytes of the decode rows (all sequences with q_len == 1,
    or the given ones)."""
    e_kv, e_q = ELEM[w.cache_dtype], ELEM[w.in_dtype]
    vis = visible_keys(w)
    offs = w.q_offsets
    sel = np.nonzero(is_decode(w))[0] if seqs is None else np.asarray(seqs)
    total = 0
    for s in sel:
        n = int(vis[offs[s]])
        b = n * w.num_kv_heads * w.head_dim * 2 * e_kv
        if w.cache_dtype == "e4m3":
            b += n * w.num_kv_heads * 2 * 4
        b += w.num_q_heads * w.head_dim * (e_q + e_q) + (-(-n // w.page_size)) * 4 + w.num_q_heads * 4
        total += b
    return int(total)


def prefill_flops(w):
    """Algorithmic flops of the prefill rows (sequences with q_len > 1)."""
    vis = visible_keys(w)
    offs = w.q_offsets
    pairs = 0
    for s in np.nonzero(w.q_lens > 1)[0]:
        pairs += int(np.sum(vis[offs[s]:offs[s + 1]]))
    return 4 * w.head_dim * w.num_q_heads * pairs


def prefill_pairs(w):
    vis = visible_keys(w)
    offs = w.q_offsets
    return int(sum(int(np.sum(vis[offs[s]:offs[s + 1]])) for s in np.nonzero(w.q_lens > 1)[0]))


def rope_bytes(w):
    e_in, e_c = ELEM[w.in_dtype], ELEM[w.cache_dtype]
    T = w.total_q
    b = T * w.num_q_heads * w.head_dim * 2 * e_in                 # q in, q out
    b += T * w.num_kv_heads * w.head_dim * 2 * (e_in + e_c)        # k, v in; cache out
    if w.cache_dtype == "e4m3":
        b += T * w.num_kv_heads * 2 * 4
    b += T * (w.rotary_dim // 2) * 8                               # table rows
    streams = len(w.mrope_sections) if w.mrope_sections is not None else (1 if w.explicit_positions else 0)
    b += T * 4 * (1 + streams)                                     # page-table entry + position ids
    return int(b)


def kv_cache_memory_bytes(layers, heads, d_head, seq_len, batch, elem_bytes=2):
    """Footprint of a K+V cache (Algenta ``kv_cache_memory_bytes``)."""
    return 2 * layers * heads * d_head * seq_len * batch * elem_bytes
