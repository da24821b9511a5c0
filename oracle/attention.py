"""Ragged scaled-dot-product attention over a paged KV cache (TEST
INFRASTRUCTURE).

Definitions followed:

* NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache" and
  ``attention_packed``: segment s spans rows offsets[s] .. offsets[s+1]-1 of
  the batch; queries align to the end of their segment's keys, so row r of q
  query rows over k keys sits at position r + k - q and sees keys from that
  position minus
  ``keys_before`` through that position plus ``keys_after``; ``keys_after=0``
  is causal; ``keys_before = w - 1`` is a window of w keys; a row without a
  visible key has an all-zero output; the forward also returns a
  log-sum-exp per (token, head).
* Algenta "Attention variant kernels", "A scalar reference, not a buffer
  kernel": the score is q.k / sqrt(d) (here an explicit ``softmax_scale``
  replaces 1/sqrt(d), as the aria_kernel ``attention_with_scale`` entry
  allows), the causal mask admits key position <= query position, and the
  softmax subtracts the row maximum before exponentiating.
* Algenta, "Ten named techniques, one scalar formula each",
  ``streaming_llm_sink_score``: StreamingLLM keeps the first few ("sink")
  keys visible besides a sliding window of recent keys.
* Algenta, "Flash attention's running state ...":
  ``grouped_query_attention_scale(32, 8) = 4`` -- each KV head serves
  Hq / Hkv query heads.

Readings taken where the pages leave a step open: query head h reads KV head
floor(h / G) with G = Hq / Hkv; ``window_left`` = keys_before and
``window_right`` = keys_after, -1 standing for the pages' None (unbounded),
window_right 0 (the default) being causal; ``sink_keys`` = n keys from the
segment's first that every row sees in addition to its band, up to the
band's right edge (sinks widen the left side only; 0 = none);
the log-sum-exp is the natural log of sum_j exp(scale * q.k_j); an empty
row has lse = -inf.

This is the plain definition: full score rows, one max, one exponent, one
sum, one division -- no tiling, no online softmax, no split.
"""

import numpy as np


def visible_range(row, q_len, kv_len, window_left, window_right=0):
    """Inclusive key range [lo, hi] visible to query row ``row`` of a segment
    with ``q_len`` query rows over ``kv_len`` keys (empty when lo > hi): from
    the row's position minus keys_before through the position plus
    keys_after, clipped to the segment's keys."""
    p = row + kv_len - q_len                    # end-aligned query position
    hi = kv_len - 1 if window_right < 0 else min(p + window_right, kv_len - 1)
    lo = 0 if window_left < 0 else max(0, p - window_left)
    return lo, hi


def visible_keys(row, q_len, kv_len, window_left, window_right=0, sink_keys=0):
    """Sorted indices of the keys visible to query row ``row``: its band
    [lo, hi] and, up to hi, the first ``sink_keys`` keys of the segment."""
    lo, hi = visible_range(row, q_len, kv_len, window_left, window_right)
    band = np.arange(lo, hi + 1) if lo <= hi else np.zeros(0, dtype=np.int64)
    if sink_keys <= 0:
        return band
    return np.union1d(np.arange(max(0, min(sink_keys, hi + 1))), band).astype(np.int64)


def attend_rows(q_rows, K, V, row_ids, q_len, kv_len, softmax_scale, window_left, window_right=0,
                sink_keys=0):
    """Attention for selected query rows of one segment and one KV head.

    q_rows [n, D] float64, K/V [kv_len, D] float64, row_ids [n] local rows.
    Returns out [n, D], lse [n].
    """
    n, d = q_rows.shape
    out = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    scores = softmax_scale * (q_rows @ K.T)     # [n, kv_len]
    for r in range(n):
        idx = visible_keys(int(row_ids[r]), q_len, kv_len, window_left, window_right, sink_keys)
        if idx.size == 0:
            continue
        s = scores[r, idx]
        m = np.max(s)
        e = np.exp(s - m)
        l = np.sum(e)
        out[r] = (e @ V[idx]) / l
        lse[r] = m + np.log(l)
    return out, lse


def ragged_paged_attention(q, q_offsets, kv_lens, cache, page_table, softmax_scale,
                           window_left=-1, rows=None, window_right=0, sink_keys=0):
    """Attention of every (or the selected) query row of a ragged batch.

    q [T, Hq, D]: float64 values of the stored queries.  ``cache`` is an
    ``oracle.paged.PagedCache``.  ``rows`` optionally restricts the
    computation to a list of global token indices (outputs of other rows are
    left zero / -inf).  Returns out [T, Hq, D] float64, lse [T, Hq] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    q_offsets = np.asarray(q_offsets, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    T, hq, d = q.shape
    hkv = cache.num_kv_heads
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.zeros((T, hq, d))
    lse = np.full((T, hq), -np.inf)
    wanted = None if rows is None else np.zeros(T, dtype=bool)
    if wanted is not None:
        wanted[np.asarray(rows, dtype=np.int64)] = True
    for s in range(len(kv_lens)):
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        q_len, kv_len = b - a, int(kv_lens[s])
        local = np.arange(q_len)
        if wanted is not None:
            local = local[wanted[a:b]]
        if q_len == 0 or local.size == 0:
            continue
        K, V = cache.gather(page_table, s, kv_len)
        for h in range(hq):
            g = h // group
            o, l = attend_rows(q[a + local, h, :], K[:, g, :], V[:, g, :], local,
                               q_len, kv_len, softmax_scale, window_left, window_right, sink_keys)
            out[a + local, h, :] = o
            lse[a + local, h] = l
    return out, lse


def dense_attention(q, k, v, softmax_scale, window_left=-1, window_right=0, sink_keys=0):
    """Single-segment attention on contiguous arrays (no pages).

    q [n_q, Hq, D], k/v [n_kv, Hkv, D] float64; end-aligned band (causal by
    default).
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, hq, d = q.shape
    n_kv, hkv, _ = k.shape
    group = hq // hkv
    out = np.zeros((n_q, hq, d))
    lse = np.full((n_q, hq), -np.inf)
    for h in range(hq):
        g = h // group
        o, l = attend_rows(q[:, h, :], k[:, g, :], v[:, g, :], np.arange(n_q),
                           n_q, n_kv, softmax_scale, window_left, window_right, sink_keys)
        out[:, h, :] = o
        lse[:, h] = l
    return out, lse


def ragged_paged_attention_backward(q, q_offsets, kv_lens, cache, page_table, softmax_scale, dout,
                                    window_left=-1, window_right=0, sink_keys=0):
    """Gradients of ``ragged_paged_attention`` (NumKong matrix-kernels page,
    ``attention_packed_gradients``: query, key and value gradients under the
    same band), from the plain definition: per row, P = softmax of the
    visible scores, out = P V; for the output gradient dO the softmax
    Jacobian gives dS_j = P_j (dO.v_j - dO.out), and
    dq = scale sum_j dS_j k_j, dk_j += scale dS_j q, dv_j += P_j dO,
    summed over the query heads sharing a KV head.

    q, dout [T, Hq, D] float64.  Returns dq [T, Hq, D] and lists dk, dv of
    per-segment [kv_len, Hkv, D] arrays.
    """
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, hq, d = q.shape
    hkv = cache.num_kv_heads
    group = hq // hkv
    dq = np.zeros_like(q)
    dk, dv = [], []
    for s in range(len(kv_lens)):
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        q_len, kv_len = b - a, int(kv_lens[s])
        K, V = cache.gather(page_table, s, kv_len)
        dK = np.zeros((kv_len, hkv, d))
        dV = np.zeros((kv_len, hkv, d))
        for r in range(q_len):
            idx = visible_keys(r, q_len, kv_len, window_left, window_right, sink_keys)
            if idx.size == 0:
                continue
            for h in range(hq):
                g = h // group
                qi, doi = q[a + r, h], dout[a + r, h]
                sc = softmax_scale * (K[idx, g] @ qi)
                e = np.exp(sc - np.max(sc))
                p = e / np.sum(e)
                o = p @ V[idx, g]
                ds = p * (V[idx, g] @ doi - doi @ o)
                dq[a + r, h] = softmax_scale * (ds @ K[idx, g])
                dK[idx, g] += softmax_scale * ds[:, None] * qi[None, :]
                dV[idx, g] += p[:, None] * doi[None, :]
        dk.append(dK)
        dv.append(dV)
    return dq, dk, dv
