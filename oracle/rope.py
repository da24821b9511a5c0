"""Rotary embedding of Q and K and the append of K/V into cache pages
(TEST INFRASTRUCTURE).

What is computed, per the pages:

* Mojo page, ``generic_fused_qk_rope_bshd_paged_ragged_kernel_api``: rotary
  embedding is applied to Q and K, the rotated Q goes to the output, and the
  keys in the paged cache are updated in place; ``input_row_offsets`` are the
  cumulative ragged row offsets; ``position_ids`` (when present) index the
  ``freqs_cis`` table; ``interleaved`` pairs adjacent (real, imaginary)
  components instead of splitting the head into halves.
* aria_kernel crate, ``rope`` (interleaved pairs), ``rope_half`` (rotate-half:
  a contiguous half of the dims pairs with the other half),
  ``rope_half_partial`` (only the first ``rotary_dim`` dims rotate) and
  ``rope_half_proportional`` (p-RoPE: the rotate-half pairing over the whole
  head, only its first pairs rotate, the others stay identity; their
  frequencies use the full head_dim denominator).
* NumKong matrix-kernels page, ``attention_rope``: every channel pair of each
  head is rotated by per-token cos/sin grids shared across heads.
* Mojo page, ``mrope_section``: M-RoPE partitions the head dimension across
  modalities.

Readings taken where the pages leave a step open:

* rotation sign: a pair (x, y) is the complex number x + iy multiplied by
  cos + i sin, so x' = x cos - y sin and y' = x sin + y cos;
* the table is ``freqs[pos][i] = (cos, sin)`` of pair i at position pos,
  float32, shape ``[max_pos, rotary_dim/2, 2]``; pairs are
  half: (i, i + R/2), interleaved: (2i, 2i+1), for i < R/2, dims >= R pass;
  half_proportional: (i, i + D/2) for i < R/2 (R = 2 x the rotated pairs),
  every other dim passes; the table's frequencies are the caller's;
* token i of segment s goes to logical slot ``kv_len[s] - q_len[s] + i``
  (``kv_len`` counts keys after the append); without position ids the
  position is that slot;
* V is stored unrotated in the same slot as K;
* M-RoPE: the sections count rotated pairs (summing to R/2, in pair order);
  each token carries one position per section, and pair i reads the table
  row of its section's position (the multimodal RoPE of vision-language
  models: temporal, height, width);
* float8 cache: one scale per (token, kv head), ``scale = fl32(absmax/448)``
  of the float64 row to be stored, codes ``e4m3(x / scale)``.

Rounding happens only where the operation stores: q_out in the input dtype,
the cache in the cache dtype.
"""

import numpy as np

from . import formats
from .paged import PagedCache


def pair_indices(rotary_dim, layout, head_dim=None):
    """Index arrays (first, second) of the rotated pairs."""
    if rotary_dim % 2:
        raise ValueError("rotary_dim must be even")
    half = rotary_dim // 2
    i = np.arange(half)
    if layout == "half":
        return i, i + half
    if layout == "interleaved":
        return 2 * i, 2 * i + 1
    if layout == "half_proportional":
        if head_dim is None or head_dim % 2 or rotary_dim > head_dim:
            raise ValueError("half_proportional needs an even head_dim >= rotary_dim")
        return i, i + head_dim // 2
    raise ValueError(layout)


def rotate(x, cos, sin, rotary_dim, layout):
    """Rotate the first ``rotary_dim`` dims of x [..., D] (float64).

    ``cos``/``sin`` have shape [..., R/2] broadcastable against x's leading
    dims; dims >= R are returned unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    a_idx, b_idx = pair_indices(rotary_dim, layout, x.shape[-1])
    out = x.copy()
    a = x[..., a_idx]
    b = x[..., b_idx]
    out[..., a_idx] = a * cos - b * sin
    out[..., b_idx] = a * sin + b * cos
    return out


def token_slots(q_offsets, kv_lens, position_ids=None):
    """Per token: (sequence, slot, position) arrays for a ragged batch."""
    q_offsets = np.asarray(q_offsets, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    total = int(q_offsets[-1])
    seq = np.empty(total, dtype=np.int64)
    slot = np.empty(total, dtype=np.int64)
    for s in range(len(kv_lens)):
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        seq[a:b] = s
        slot[a:b] = kv_lens[s] - (b - a) + np.arange(b - a)
    pos = slot.copy() if position_ids is None else np.asarray(position_ids, dtype=np.int64)
    return seq, slot, pos


def pair_positions(position_ids, sections, rotary_dim):
    """Position of every (token, rotated pair) under M-RoPE: position_ids
    [n_sections, T], sections = rotated pairs per section (sum R/2); pair i
    takes the position of the section that holds it.  Returns [T, R/2]."""
    position_ids = np.asarray(position_ids, dtype=np.int64)
    sections = [int(x) for x in sections]
    if sum(sections) != rotary_dim // 2 or position_ids.shape[0] != len(sections):
        raise ValueError("sections must count R/2 pairs, one position stream each")
    sec_of_pair = np.repeat(np.arange(len(sections)), sections)           # [R/2]
    return position_ids[sec_of_pair, :].T                                # [T, R/2]


def rope_qk_write_paged(q, k, v, in_dtype, q_offsets, kv_lens, position_ids,
                        freqs, rotary_dim, layout, cache: PagedCache, page_table, mrope_sections=None):
    """Rotate Q and K, store K/V into the cache.

    q [T, Hq, D], k/v [T, Hkv, D]: float64 values of the stored inputs.
    freqs [max_pos, R/2, 2]: the float32 table (values widened).
    With ``mrope_sections`` (rotated pairs per section), position_ids is
    [n_sections, T] and pair i rotates by its section's position.
    Returns (q_out as stored, updated copy of the cache).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    freqs = np.asarray(freqs, dtype=np.float64)
    if mrope_sections is None:
        seq, slot, pos = token_slots(q_offsets, kv_lens, position_ids)
        cos = freqs[pos, :, 0][:, None, :]      # [T, 1, R/2] shared across heads
        sin = freqs[pos, :, 1][:, None, :]
    else:
        seq, slot, _ = token_slots(q_offsets, kv_lens)
        pp = pair_positions(position_ids, mrope_sections, rotary_dim)    # [T, R/2]
        pair = np.arange(rotary_dim // 2)[None, :]
        cos = freqs[pp, pair, 0][:, None, :]
        sin = freqs[pp, pair, 1][:, None, :]
    q_rot = rotate(q, cos, sin, rotary_dim, layout)
    k_rot = rotate(k, cos, sin, rotary_dim, layout)
    q_out = formats.storage_round(q_rot, in_dtype)

    out = cache.copy()
    for t in range(q.shape[0]):
        for h in range(k.shape[1]):
            if cache.dtype == "e4m3":
                kc, ks = formats.fp8_quantize(k_rot[t, h])
                vc, vs = formats.fp8_quantize(v[t, h])
                out.store(page_table, seq[t], slot[t], h,
                          formats.e4m3_value(kc), formats.e4m3_value(vc), ks, vs)
            else:
                out.store(page_table, seq[t], slot[t], h,
                          formats.storage_round(k_rot[t, h], cache.dtype),
                          formats.storage_round(v[t, h], cache.dtype))
    return q_out, out
