"""Log-sum-exp merge of partial attention states (TEST INFRASTRUCTURE).

Algenta "Attention variant kernels", "Flash attention's running state
reproduces the same softmax": a pass over keys keeps a running maximum m, a
running normaliser l and a running (unnormalised) output o; when the maximum
rises, l and o are rescaled by exp(old_max - new_max); the result is o / l and
it equals the plain stable softmax.  A partial state over a chunk of keys is
equivalently (o_c / l_c, lse_c = m_c + ln l_c); merging chunks with the same
rescaling gives, for chunks i of one (row, head):

    M   = max_i lse_i
    w_i = exp(lse_i - M)
    lse = M + ln(sum_i w_i)
    out = sum_i w_i * out_i / sum_i w_i

(the chunk outputs are already normalised, so w_i = l_i exp(m_i - M)).
Reading for empty input: if every lse_i is -inf the row saw no key and the
result is out = 0, lse = -inf (NumKong: rows that see no key return zeros).
"""

import numpy as np


def lse_merge(partial_out, partial_lse, merge_offsets):
    """partial_out [n_part, H, D], partial_lse [n_part, H] (natural log),
    merge_offsets [R+1]: partials merge_offsets[r]..merge_offsets[r+1]-1 form
    row r.  Returns out [R, H, D] float64, lse [R, H] float64."""
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    offs = np.asarray(merge_offsets, dtype=np.int64)
    rows = len(offs) - 1
    _, h, d = po.shape
    out = np.zeros((rows, h, d))
    lse = np.full((rows, h), -np.inf)
    for r in range(rows):
        a, b = int(offs[r]), int(offs[r + 1])
        if a == b:
            continue
        chunk_lse = pl[a:b]                               # [n, H]
        M = np.max(chunk_lse, axis=0)                      # [H]
        live = np.isfinite(M)
        Ms = np.where(live, M, 0.0)
        w = np.where(np.isfinite(chunk_lse), np.exp(chunk_lse - Ms), 0.0)
        tot = np.sum(w, axis=0)                            # [H]
        num = np.einsum("nh,nhd->hd", w, po[a:b])
        safe = np.where(live, tot, 1.0)
        out[r] = np.where(live[:, None], num / safe[:, None], 0.0)
        lse[r] = np.where(live, Ms + np.log(safe), -np.inf)
    return out, lse


def online_softmax_trace(scores, values):
    """The running state (m, l, o) after each key, one key at a time, as the
    Algenta page steps it (starting from m = -1e9, l = 0, o = 0), followed by
    the final o / l.  ``values`` may be scalars or vectors."""
    m, l, o = -1e9, 0.0, 0.0
    trace = []
    for s, v in zip(scores, values):
        new_m = max(m, s)
        corr = np.exp(m - new_m)
        p = np.exp(s - new_m)
        l = l * corr + p
        o = o * corr + p * np.asarray(v, dtype=np.float64)
        m = new_m
        trace.append((m, l, o))
    return trace, o / l
