"""Pure-Python brute force of the same definitions, for tiny inputs (TEST
INFRASTRUCTURE).

Plain loops with ``math.exp``/``math.log``/``math.fsum`` and nested lists;
no numpy arithmetic.  Used to cross-check the numpy oracle.  The definitions
are the ones cited in ``oracle.attention``, ``oracle.rope`` and
``oracle.merge``; the paged cache is read slot by slot through the page
table.
"""

import math


def rope_row(x, cos_row, sin_row, rotary_dim, layout):
    """Rotate one head vector (list of floats) by one position's cos/sin."""
    out = list(x)
    half = rotary_dim // 2
    for i in range(half):
        if layout == "half":
            a, b = i, i + half
        elif layout == "half_proportional":          # pairs span the whole head
            a, b = i, i + len(x) // 2
        else:
            a, b = 2 * i, 2 * i + 1
        c, s = cos_row[i], sin_row[i]
        out[a] = x[a] * c - x[b] * s
        out[b] = x[a] * s + x[b] * c
    return out


def attention_row(q, keys, values, scale):
    """One query against a list of visible keys/values -> (out, lse)."""
    if not keys:
        return [0.0] * len(q), -math.inf
    scores = [scale * math.fsum(qi * ki for qi, ki in zip(q, k)) for k in keys]
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    l = math.fsum(e)
    out = [math.fsum(e[j] * values[j][d] for j in range(len(keys))) / l
           for d in range(len(q))]
    return out, m + math.log(l)


def ragged_attention(q, q_offsets, kv_lens, keys, values, scale, window_left=-1, window_right=0,
                     sink_keys=0):
    """q: list over tokens of list over heads of vectors; keys/values: list
    over sequences of list over slots of list over kv heads of vectors.
    Returns (out, lse) nested lists [T][Hq][D], [T][Hq]."""
    hq = len(q[0]) if q else 0
    hkv = len(keys[0][0]) if keys and keys[0] else 1
    group = hq // hkv if hkv else 1
    out, lse = [], []
    for s in range(len(kv_lens)):
        a, b = q_offsets[s], q_offsets[s + 1]
        q_len, kv_len = b - a, kv_lens[s]
        for r in range(q_len):
            p = r + kv_len - q_len
            lo = 0 if window_left < 0 else max(0, p - window_left)
            hi = kv_len - 1 if window_right < 0 else min(p + window_right, kv_len - 1)
            seen = [j for j in range(kv_len) if j <= hi and (j < sink_keys or j >= lo)]
            row_out, row_lse = [], []
            for h in range(hq):
                g = h // group
                ks = [keys[s][j][g] for j in seen]
                vs = [values[s][j][g] for j in seen]
                o, l = attention_row(q[a + r][h], ks, vs, scale)
                row_out.append(o)
                row_lse.append(l)
            out.append(row_out)
            lse.append(row_lse)
    return out, lse


def merge_states(states):
    """Merge a list of (out_vector, lse) partial states of one (row, head)."""
    lses = [l for _, l in states if l != -math.inf]
    if not lses:
        return [0.0] * len(states[0][0]), -math.inf
    M = max(lses)
    ws = [math.exp(l - M) if l != -math.inf else 0.0 for _, l in states]
    tot = math.fsum(ws)
    d = len(states[0][0])
    out = [math.fsum(w * o[i] for w, (o, _) in zip(ws, states)) / tot for i in range(d)]
    return out, M + math.log(tot)
