"""Packing ragged K/V token matrices into the paged cache (TEST
INFRASTRUCTURE).

NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache" and
``attention_pack``: one pack, built once, serves many attention calls.
Segment s's input slot is rows key_offsets[s] .. key_offsets[s+1]-1; the
first kept_s rows of it enter the pack, kept_s being ``key_lengths[s]``, or
the slot's size when no lengths are given.

The pack's layout is opaque on the page; here it is the library's paged
cache (``paged``).  Readings taken where the page leaves a step open:

* pages are assigned in segment order: segment s takes pages
  first_s .. first_s + ceil(kept_s / P) - 1 with first_s the sum of the page
  counts of segments 0..s-1;
* a kept length is clamped to [0, slot size] (the page has a segment hold
  fewer keys than its slot, never more) and to the stated maximum;
* keys are stored as given (no rotation): rounded once to the cache type, an
  e4m3 row with its scale absmax/448 as the append step stores it;
* attention over the pack is the ragged attention with kv_len = kept length
  (queries aligned to the end of each segment's kept keys).
"""

import numpy as np

from . import formats
from .paged import PagedCache


def kept_lengths(key_offsets, key_lengths=None, max_key_len=None):
    """Kept keys per segment (int64 [B])."""
    offs = np.asarray(key_offsets, dtype=np.int64)
    slot = offs[1:] - offs[:-1]
    kept = slot.copy() if key_lengths is None else np.minimum(np.maximum(np.asarray(key_lengths, np.int64), 0), slot)
    if max_key_len is not None:
        kept = np.minimum(kept, max_key_len)
    return kept


def page_assignment(kept, page_size):
    """First page and page count of every segment, in segment order."""
    counts = -(-np.asarray(kept, dtype=np.int64) // page_size)
    first = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    return first, counts


def attention_pack(k, v, key_offsets, key_lengths, cache_dtype, page_size, num_pages=None, max_key_len=None):
    """k, v: float64 values [rows, Hkv, D] (the inputs as given).  Returns
    (cache, page_table [B, stride] int64, kept [B])."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows, hkv, d = k.shape
    kept = kept_lengths(key_offsets, key_lengths, max_key_len)
    first, counts = page_assignment(kept, page_size)
    total = int(counts.sum())
    n = total if num_pages is None else num_pages
    if n < total:
        raise ValueError("cache smaller than the pack")
    stride = max(1, int(counts.max()) if len(counts) else 1)
    table = np.zeros((len(kept), stride), dtype=np.int64)
    for s in range(len(kept)):
        table[s, :counts[s]] = first[s] + np.arange(counts[s])
    cache = PagedCache(cache_dtype, max(n, 1), hkv, page_size, d)
    offs = np.asarray(key_offsets, dtype=np.int64)
    for s in range(len(kept)):
        for j in range(int(kept[s])):
            row = offs[s] + j
            for h in range(hkv):
                if cache_dtype == "e4m3":
                    kc, ks = formats.fp8_quantize(k[row, h])
                    vc, vs = formats.fp8_quantize(v[row, h])
                    cache.store(table, s, j, h, formats.e4m3_value(kc), formats.e4m3_value(vc), ks, vs)
                else:
                    cache.store(table, s, j, h, formats.storage_round(k[row, h], cache_dtype),
                                formats.storage_round(v[row, h], cache_dtype))
    return cache, table, kept
