"""The paged KV cache of ``include/nk.h``, addressed element by element
(TEST INFRASTRUCTURE).

Layout (one layer):

* K pages  ``[num_pages][num_kv_heads][head_dim/(32*NK)][page_size][32*NK]``
  with NK = 2 for e4m3 and 1 otherwise -- within a page, for one head, K is
  stored in blocks of 32*NK dimensions, token after token; a token's row of
  a block is 4 runs of NK*8 elements, run g holding dims 8g..8g+7 of each
  32-dim half (for NK = 1: dims 32b..32b+31 in order).
* V pages  ``[num_pages][num_kv_heads][page_size/16][head_dim/(16*NV)][64][4*NV]``
  with NV = 4 / element bytes (f32 1, bf16 2, e4m3 4) -- within a page, for
  one head, each block of 16 tokens is a sequence of 16-byte runs; run
  ``16*g + l`` of dim group ``c`` holds tokens ``4g..4g+3`` of the block for
  the dims ``16*(c*NV + j) + l``, ``j = 0..NV-1`` (dim-major within the run).
* fp8 scales (K and V separately) ``[num_pages][num_kv_heads][page_size]``.
* ``page_table[s][p]`` is the physical page holding logical slots
  ``p*page_size .. p*page_size + page_size - 1`` of sequence ``s``.

The pages define a cache whose pages a caller packs once and reads many times
(NumKong matrix-kernels page, "Attention with a Pre-Packed KV-Cache"), updated
in place by the fused RoPE step (Mojo page,
``generic_fused_qk_rope_bshd_paged_ragged_kernel_api``, ``kv_collection``).
The physical layout is not fixed by the pages; the one above is this
library's.

The oracle keeps the cache as float64 *stored values*: for ``f32`` and
``bf16`` the element values, for ``e4m3`` the values of the codes (unscaled)
plus the per-slot scales, with K held token-major ([page][head][slot][dim]);
``from_storage`` / ``to_storage`` convert to and from the raw bytes of the
layout above.
"""

import numpy as np

from . import formats

DTYPES = ("f32", "bf16", "e4m3")


class PagedCache:
    def __init__(self, dtype, num_pages, num_kv_heads, page_size, head_dim):
        if dtype not in DTYPES:
            raise ValueError(dtype)
        self.dtype = dtype
        self.num_pages = num_pages
        self.num_kv_heads = num_kv_heads
        self.page_size = page_size
        self.head_dim = head_dim
        self.k = np.full((num_pages, num_kv_heads, page_size, head_dim), np.nan)
        self.v = np.full((num_pages, num_kv_heads, head_dim, page_size), np.nan)
        if dtype == "e4m3":
            self.k_scale = np.full((num_pages, num_kv_heads, page_size), np.nan)
            self.v_scale = np.full((num_pages, num_kv_heads, page_size), np.nan)
        else:
            self.k_scale = self.v_scale = None

    def copy(self):
        c = PagedCache(self.dtype, self.num_pages, self.num_kv_heads,
                       self.page_size, self.head_dim)
        c.k, c.v = self.k.copy(), self.v.copy()
        if self.k_scale is not None:
            c.k_scale, c.v_scale = self.k_scale.copy(), self.v_scale.copy()
        return c

    # -- raw storage <-> stored values ------------------------------------
    @classmethod
    def from_storage(cls, dtype, k_pages, v_pages, k_scales=None, v_scales=None):
        """Build from raw arrays: float32 (f32), uint16 bit patterns (bf16)
        or uint8 codes (e4m3), shaped as the layout above."""
        n, h, nb, p, blk = k_pages.shape
        if blk != 32 * k_block_halves(dtype):
            raise ValueError("K pages must be [num_pages][heads][head_dim/(32*NK)][page_size][32*NK]")
        d = nb * blk
        c = cls(dtype, n, h, p, d)
        nv = v_run_width(dtype)
        if tuple(v_pages.shape) != (n, h, p // 16, d // (16 * nv), 64, 4 * nv):
            raise ValueError("V pages must be [num_pages][heads][page_size/16][head_dim/(16*NV)][64][4*NV]")
        c.k = _decode(dtype, k_storage_to_logical(dtype, np.asarray(k_pages)))
        c.v = _decode(dtype, v_storage_to_logical(dtype, np.asarray(v_pages)))
        if dtype == "e4m3":
            c.k_scale = np.asarray(k_scales, dtype=np.float32).astype(np.float64)
            c.v_scale = np.asarray(v_scales, dtype=np.float32).astype(np.float64)
        return c

    def to_storage(self):
        """Raw arrays (k_pages, v_pages, k_scales, v_scales); unwritten slots
        (NaN) become the dtype's NaN pattern, scales NaN."""
        n, h, p, d = self.k.shape
        k = k_logical_to_storage(self.dtype, _encode(self.dtype, self.k))
        v = v_logical_to_storage(self.dtype, _encode(self.dtype, self.v))
        if self.dtype == "e4m3":
            return k, v, self.k_scale.astype(np.float32), self.v_scale.astype(np.float32)
        return k, v, None, None

    # -- logical slot access -------------------------------------------------
    def locate(self, page_table, seq, slot):
        """Logical slot of a sequence -> (physical page, offset in page)."""
        page = int(page_table[seq][slot // self.page_size])
        return page, slot % self.page_size

    def store(self, page_table, seq, slot, head, k_vals, v_vals, k_scale=None, v_scale=None):
        """Store one (token, kv head) row of stored values into its slot."""
        page, off = self.locate(page_table, seq, slot)
        self.k[page, head, off, :] = k_vals
        self.v[page, head, :, off] = v_vals
        if self.dtype == "e4m3":
            self.k_scale[page, head, off] = k_scale
            self.v_scale[page, head, off] = v_scale

    def gather(self, page_table, seq, length):
        """Dequantised K and V of slots 0..length-1 of a sequence, as float64
        arrays [length, num_kv_heads, head_dim]."""
        slots = np.arange(length)
        pages = np.asarray(page_table[seq])[slots // self.page_size].astype(np.int64)
        offs = slots % self.page_size
        K = self.k[pages, :, offs, :]            # [length, heads, head_dim]
        V = self.v[pages, :, :, offs]            # [length, heads, head_dim]
        if self.dtype == "e4m3":
            K = K * self.k_scale[pages, :, offs][:, :, None]
            V = V * self.v_scale[pages, :, offs][:, :, None]
        return K, V


def k_block_halves(dtype):
    """NK: 32-dim halves per K block (2 for e4m3, else 1)."""
    return 2 if dtype == "e4m3" else 1


def k_storage_to_logical(dtype, raw):
    """[n][h][D/(32 NK)][P][32 NK] -> token-major [n][h][P][D]."""
    nk = k_block_halves(dtype)
    n, h, nb, p, row = raw.shape
    if row != 32 * nk:
        raise ValueError("K pages must be [num_pages][heads][head_dim/(32*NK)][page_size][32*NK]")
    x = raw.reshape(n, h, nb, p, 4, nk, 8)                  # n h s t g half e
    x = np.transpose(x, (0, 1, 3, 2, 5, 4, 6))              # n h t s half g e
    return x.reshape(n, h, p, nb * nk * 32)


def k_logical_to_storage(dtype, k):
    """Inverse of k_storage_to_logical."""
    nk = k_block_halves(dtype)
    n, h, p, d = k.shape
    x = k.reshape(n, h, p, d // (32 * nk), nk, 4, 8)         # n h t s half g e
    x = np.transpose(x, (0, 1, 3, 2, 5, 4, 6))               # n h s t g half e
    return np.ascontiguousarray(x).reshape(n, h, d // (32 * nk), p, 32 * nk)


def v_run_width(dtype):
    """NV: 16-dim groups per 16-byte V run (4 / element bytes)."""
    return {"f32": 1, "bf16": 2, "e4m3": 4}[dtype]


def v_storage_to_logical(dtype, raw):
    """[n][h][P/16][D/(16 NV)][64][4 NV] -> [n][h][D][P] (same element type).

    Axes after splitting 64 into (g, l) and 4 NV into (j, t4): token
    16*sb + 4*g + t4, dim 16*(c*NV + j) + l."""
    nv = v_run_width(dtype)
    n, h, nsb, nc, lanes, run = raw.shape
    if lanes != 64 or run != 4 * nv:
        raise ValueError("V pages must be [num_pages][heads][page_size/16][head_dim/(16*NV)][64][4*NV]")
    x = raw.reshape(n, h, nsb, nc, 4, 16, nv, 4)            # n h sb c g l j t4
    x = np.transpose(x, (0, 1, 3, 6, 5, 2, 4, 7))           # n h c j l sb g t4
    return x.reshape(n, h, nc * nv * 16, nsb * 16)


def v_logical_to_storage(dtype, v):
    """Inverse of v_storage_to_logical."""
    nv = v_run_width(dtype)
    n, h, d, p = v.shape
    x = v.reshape(n, h, d // (16 * nv), nv, 16, p // 16, 4, 4)   # n h c j l sb g t4
    x = np.transpose(x, (0, 1, 5, 2, 6, 4, 3, 7))                # n h sb c g l j t4
    return np.ascontiguousarray(x).reshape(n, h, p // 16, d // (16 * nv), 64, 4 * nv)


def _decode(dtype, raw):
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return formats.bf16_value(raw.view(np.uint16) if raw.dtype != np.uint16 else raw)
    return formats.e4m3_value(raw.view(np.uint8) if raw.dtype != np.uint8 else raw)


def _encode(dtype, vals):
    if dtype == "f32":
        return vals.astype(np.float32)
    if dtype == "bf16":
        return formats.bf16_bits(vals)
    return formats.e4m3_code(vals)
