"""Python binding of libnk.so (ctypes): argument marshalling only.

Every function here checks devices, dtypes, shapes and contiguity of torch
tensors, passes raw device pointers and the current HIP stream to the C ABI
declared in ``include/nk.h``, and raises ``NKError`` on a non-zero status.
All computation happens in the library's HIP kernels; if the library is not
built, importing works but every call raises.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnk.so")

NK_F32, NK_BF16, NK_E4M3 = 0, 1, 2
NK_ROPE_HALF, NK_ROPE_INTERLEAVED, NK_ROPE_HALF_PROPORTIONAL = 0, 1, 2
NK_OK, NK_ERR_INVALID_ARG, NK_ERR_UNSUPPORTED, NK_ERR_WORKSPACE, NK_ERR_DEVICE = 0, 1, 2, 3, 4

EXPORTS = ("nk_rope_qk_write_paged", "nk_rope_qk_write_paged_mrope", "nk_ragged_paged_attention", "nk_ragged_paged_attention_band",
           "nk_ragged_paged_attention_workspace_size", "nk_ragged_paged_attention_split_tokens",
           "nk_attention_lse_merge", "nk_status_string", "nk_version", "nk_profile_enable",
           "nk_profile_reset", "nk_profile_read", "nk_attention_pack", "nk_ragged_paged_attention_backward",
           "nk_ragged_paged_attention_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20       # NK_NOALLOC_SCRATCH_BYTES


class NKError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class nk_paged_kv_t(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("page_table_stride", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ragged_paged_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, sz, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        cache_p = ctypes.POINTER(nk_paged_kv_t)
        L.nk_rope_qk_write_paged.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                             i32, i32, i32, cache_p, vp]
        L.nk_rope_qk_write_paged.restype = ctypes.c_int
        L.nk_rope_qk_write_paged_mrope.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                                   i32, i32, i32, cache_p, vp]
        L.nk_rope_qk_write_paged_mrope.restype = ctypes.c_int
        L.nk_ragged_paged_attention.argtypes = [vp, i32, vp, vp, cache_p, f32, i32, vp, vp, i32,
                                                i32, i32, i32, i32, i32, vp, sz, vp]
        L.nk_ragged_paged_attention.restype = ctypes.c_int
        L.nk_ragged_paged_attention_band.argtypes = [vp, i32, vp, vp, cache_p, f32, i32, i32, i32, vp, vp, i32,
                                                     i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.nk_ragged_paged_attention_band.restype = ctypes.c_int
        L.nk_ragged_paged_attention_noalloc.argtypes = [vp, i32, vp, vp, cache_p, f32, i32, i32, i32, vp, vp, i32,
                                                        i32, i32, i32, i32, i32, i32, vp]
        L.nk_ragged_paged_attention_noalloc.restype = ctypes.c_int
        L.nk_ragged_paged_attention_workspace_size.argtypes = [i32] * 11
        L.nk_ragged_paged_attention_workspace_size.restype = sz
        L.nk_ragged_paged_attention_split_tokens.argtypes = [i32] * 7
        L.nk_ragged_paged_attention_split_tokens.restype = i32
        L.nk_attention_lse_merge.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, vp, vp]
        L.nk_attention_lse_merge.restype = ctypes.c_int
        L.nk_status_string.argtypes = [ctypes.c_int]
        L.nk_status_string.restype = ctypes.c_char_p
        L.nk_version.restype = ctypes.c_int
        L.nk_attention_pack.argtypes = [vp, vp, i32, vp, vp, cache_p, vp, i32, i32, vp]
        L.nk_attention_pack.restype = ctypes.c_int
        L.nk_ragged_paged_attention_backward.argtypes = [vp, i32, vp, vp, cache_p, f32, i32, i32, i32, vp, vp, vp,
                                                         vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.nk_ragged_paged_attention_backward.restype = ctypes.c_int
        L.nk_profile_enable.argtypes = [ctypes.c_int]
        L.nk_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
        _lib = L
    return _lib


def status_string(status):
    return lib().nk_status_string(int(status)).decode()


def _check(status, where):
    if status != NK_OK:
        raise NKError(status, where)


def _dtype_code(t):
    if t == torch.float32:
        return NK_F32
    if t == torch.bfloat16:
        return NK_BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return NK_E4M3
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors must share one device, got {devs}")
    d = devs.pop()
    if d.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return d


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


class PagedKVCache:
    """One layer's paged cache (device tensors in the layout of nk.h).

    k_pages [num_pages, Hkv, D/(32 NK), P, 32 NK] (NK 2 for e4m3, else 1),
    v_pages [num_pages, Hkv, P/16,
    D/(16 NV), 64, 4 NV] with NV = 4 / element bytes (float32, bfloat16 or
    uint8 e4m3 codes), k_scales/v_scales [num_pages, Hkv, P] float32 for
    e4m3, page_table [num_seqs, stride] int32.
    """

    def __init__(self, k_pages, v_pages, page_table, k_scales=None, v_scales=None):
        n, h, nb, p, blk = k_pages.shape
        nk = 2 if k_pages.element_size() == 1 else 1
        d = nb * blk
        if blk != 32 * nk:
            raise ValueError("k_pages must be [num_pages, heads, head_dim/(32*NK), page_size, 32*NK]")
        nv = 4 // k_pages.element_size()
        if d % (16 * nv) or p % 16 or tuple(v_pages.shape) != (n, h, p // 16, d // (16 * nv), 64, 4 * nv):
            raise ValueError("v_pages must be [num_pages, heads, page_size/16, head_dim/(16*NV), 64, 4*NV]")
        if k_pages.dtype != v_pages.dtype:
            raise TypeError("K and V pages must share a dtype")
        self.dtype = _dtype_code(k_pages.dtype)
        if self.dtype == NK_E4M3 and (k_scales is None or v_scales is None):
            raise ValueError("e4m3 caches need k_scales and v_scales")
        _i32(page_table, "page_table")
        _dev(k_pages, v_pages, page_table, k_scales, v_scales)
        self.k_pages, self.v_pages, self.page_table = k_pages, v_pages, page_table
        self.k_scales, self.v_scales = k_scales, v_scales
        self.num_pages, self.num_kv_heads, self.page_size, self.head_dim = n, h, p, d

    def struct(self):
        return nk_paged_kv_t(self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                             None if self.k_scales is None else self.k_scales.data_ptr(),
                             None if self.v_scales is None else self.v_scales.data_ptr(),
                             self.dtype, self.num_pages, self.page_size, self.num_kv_heads,
                             self.head_dim, self.page_table.data_ptr(),
                             self.page_table.shape[1] if self.page_table.dim() == 2 else 0)


def rope_qk_write_paged(q, k, v, q_offsets, kv_lens, freqs, cache, rotary_dim, layout="half",
                        position_ids=None, q_out=None, stream=None, mrope_sections=None):
    """Rotate q and k by ``freqs`` [max_pos, R/2, 2] and append k/v to the
    cache; returns q_out ([T, Hq, D], may be q itself).  With
    ``mrope_sections`` (rotated pairs per section, multiples of 8 summing to
    R/2), position_ids is [n_sections, T] and each section of pairs rotates
    by its own positions."""
    T, hq, d = q.shape
    if q_out is None:
        q_out = torch.empty_like(q)
    if k.shape != (T, cache.num_kv_heads, d) or v.shape != k.shape or q_out.shape != q.shape:
        raise ValueError("q/k/v shapes disagree with the cache")
    if not (q.dtype == k.dtype == v.dtype == q_out.dtype):
        raise TypeError("q, k, v, q_out must share a dtype")
    if freqs.dtype != torch.float32 or freqs.dim() != 3:
        raise TypeError("freqs must be float32 [max_pos, R/2, 2]")
    _i32(q_offsets, "q_offsets"), _i32(kv_lens, "kv_lens")
    if position_ids is not None:
        _i32(position_ids, "position_ids")
    _dev(q, k, v, q_out, q_offsets, kv_lens, position_ids, freqs, cache.k_pages)
    lay = {"half": NK_ROPE_HALF, "interleaved": NK_ROPE_INTERLEAVED,
           "half_proportional": NK_ROPE_HALF_PROPORTIONAL}[layout]
    c = cache.struct()
    if mrope_sections is None:
        st = lib().nk_rope_qk_write_paged(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(q_out),
                                          _ptr(q_offsets), _ptr(kv_lens), _ptr(position_ids), _ptr(freqs),
                                          freqs.shape[0], rotary_dim, lay, kv_lens.shape[0], T, hq,
                                          ctypes.byref(c), _stream(stream))
        _check(st, "nk_rope_qk_write_paged")
        return q_out
    if position_ids is None or position_ids.shape != (len(mrope_sections), T):
        raise ValueError("M-RoPE needs position_ids [n_sections, T]")
    sec = (ctypes.c_int32 * len(mrope_sections))(*[int(x) for x in mrope_sections])
    st = lib().nk_rope_qk_write_paged_mrope(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(q_out),
                                            _ptr(q_offsets), _ptr(kv_lens), _ptr(position_ids),
                                            len(mrope_sections), ctypes.cast(sec, ctypes.c_void_p), _ptr(freqs),
                                            freqs.shape[0], rotary_dim, lay, kv_lens.shape[0], T, hq,
                                            ctypes.byref(c), _stream(stream))
    _check(st, "nk_rope_qk_write_paged_mrope")
    return q_out


def workspace_size(q_dtype, cache, num_seqs, total_q, max_q_len, max_kv_len, num_q_heads,
                   window_left=-1, kv_split_tokens=0):
    return int(lib().nk_ragged_paged_attention_workspace_size(
        _dtype_code(q_dtype), cache.dtype, num_seqs, total_q, max_q_len, max_kv_len, num_q_heads,
        cache.num_kv_heads, cache.head_dim, window_left, kv_split_tokens))


def split_tokens(cache, num_seqs, max_kv_len, num_q_heads, window_left=-1, kv_split_tokens=0):
    return int(lib().nk_ragged_paged_attention_split_tokens(
        num_seqs, max_kv_len, num_q_heads, cache.num_kv_heads, cache.head_dim, window_left,
        kv_split_tokens))


def ragged_paged_attention(q, q_offsets, kv_lens, cache, softmax_scale, max_q_len, max_kv_len,
                           window_left=-1, out=None, lse=None, kv_split_tokens=0, workspace=None,
                           stream=None, window_right=0, sink_keys=0, min_q_len=0):
    """GQA attention of q [T, Hq, D] over the cache under the band
    [position - window_left, position + window_right] (-1 = unbounded side;
    window_right 0, the default, is causal), plus the segment's first
    ``sink_keys`` keys up to the band's right edge; returns (out, lse).  ``lse`` is
    filled when given (float32 [T, Hq]); ``workspace`` is allocated here when
    not given."""
    T, hq, d = q.shape
    B = kv_lens.shape[0]
    if out is None:
        out = torch.empty_like(q)
    _i32(q_offsets, "q_offsets"), _i32(kv_lens, "kv_lens")
    _dev(q, q_offsets, kv_lens, out, lse, cache.k_pages, workspace)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is not None and (lse.shape != (T, hq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [T, Hq]")
    need = workspace_size(q.dtype, cache, B, T, max_q_len, max_kv_len, hq, window_left, kv_split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cache.struct()
    st = lib().nk_ragged_paged_attention_band(_ptr(q), _dtype_code(q.dtype), _ptr(q_offsets), _ptr(kv_lens),
                                              ctypes.byref(c), float(softmax_scale), int(window_left),
                                              int(window_right), int(sink_keys), _ptr(out), _ptr(lse), B, T,
                                              int(min_q_len), int(max_q_len), int(max_kv_len), hq,
                                              int(kv_split_tokens), _ptr(workspace),
                                              ws_bytes, _stream(stream))
    _check(st, "nk_ragged_paged_attention_band")
    return out, lse


def ragged_paged_attention_noalloc(q, q_offsets, kv_lens, cache, softmax_scale, max_q_len, max_kv_len,
                                   window_left=-1, out=None, lse=None, kv_split_tokens=0, stream=None,
                                   window_right=0, sink_keys=0, min_q_len=0):
    """ragged_paged_attention through the entry point that takes no
    workspace (the library's static per-device scratch); ``out`` is allocated
    here when not given (the C call itself allocates nothing)."""
    T, hq, d = q.shape
    B = kv_lens.shape[0]
    if out is None:
        out = torch.empty_like(q)
    _i32(q_offsets, "q_offsets"), _i32(kv_lens, "kv_lens")
    _dev(q, q_offsets, kv_lens, out, lse, cache.k_pages)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse is not None and (lse.shape != (T, hq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [T, Hq]")
    c = cache.struct()
    st = lib().nk_ragged_paged_attention_noalloc(_ptr(q), _dtype_code(q.dtype), _ptr(q_offsets), _ptr(kv_lens),
                                                 ctypes.byref(c), float(softmax_scale), int(window_left),
                                                 int(window_right), int(sink_keys), _ptr(out), _ptr(lse), B, T,
                                                 int(min_q_len), int(max_q_len), int(max_kv_len), hq,
                                                 int(kv_split_tokens), _stream(stream))
    _check(st, "nk_ragged_paged_attention_noalloc")
    return out, lse


def attention_lse_merge(partial_out, partial_lse, merge_offsets, out, lse_out=None, stream=None):
    """Merge partial states [n, H, D] / [n, H] into rows given by
    merge_offsets [R+1]; writes out [R, H, D] (float32 or bf16)."""
    n, h, d = partial_out.shape
    R = merge_offsets.shape[0] - 1
    if partial_out.dtype != torch.float32 or partial_lse.dtype != torch.float32:
        raise TypeError("partials must be float32")
    _i32(merge_offsets, "merge_offsets")
    _dev(partial_out, partial_lse, merge_offsets, out, lse_out)
    st = lib().nk_attention_lse_merge(_ptr(partial_out), _ptr(partial_lse), _ptr(merge_offsets), R, h, d,
                                      _ptr(out), _dtype_code(out.dtype), _ptr(lse_out), _stream(stream))
    _check(st, "nk_attention_lse_merge")
    return out, lse_out


def attention_pack(k, v, key_offsets, key_lengths=None, page_size=16, cache_dtype=None, max_key_len=None,
                   num_pages=None, stream=None):
    """Pack ragged K/V rows [rows, Hkv, D] into a new paged cache: the first
    ``key_lengths[s]`` rows (all of them without lengths) of segment s's
    rows ``key_offsets[s]`` .. ``key_offsets[s+1]`` - 1 enter the pack.  Returns (cache, kv_lens, max_key_len); attention
    over it is ``ragged_paged_attention(q, q_offsets, kv_lens, cache, ...)``.
    ``cache_dtype`` is "f32", "bf16" or "e4m3" (default: the input's type).
    When ``max_key_len`` or ``num_pages`` is not given it is read from the
    lengths (a device-to-host copy)."""
    rows, hkv, d = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must share shape and dtype")
    _i32(key_offsets, "key_offsets")
    if key_lengths is not None:
        _i32(key_lengths, "key_lengths")
    _dev(k, v, key_offsets, key_lengths)
    B = key_offsets.shape[0] - 1
    cdt = cache_dtype or ("f32" if k.dtype == torch.float32 else "bf16")
    if max_key_len is None or num_pages is None:
        slots = (key_offsets[1:] - key_offsets[:-1]).cpu()
        kept = slots if key_lengths is None else torch.minimum(torch.clamp(key_lengths.cpu(), min=0), slots)
        if max_key_len is None:
            max_key_len = int(kept.max()) if B > 0 else 0
        kept = torch.clamp(kept, max=max_key_len)
        if num_pages is None:
            num_pages = int(((kept + page_size - 1) // page_size).sum())
    num_pages = max(int(num_pages), 1)
    stride = max(1, -(-int(max_key_len) // page_size))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[cdt]
    nk_ = 2 if cdt == "e4m3" else 1
    nv = {"f32": 1, "bf16": 2, "e4m3": 4}[cdt]
    dev = k.device
    kp = torch.empty(num_pages, hkv, d // (32 * nk_), page_size, 32 * nk_, dtype=tdt, device=dev)
    vp = torch.empty(num_pages, hkv, page_size // 16, d // (16 * nv), 64, 4 * nv, dtype=tdt, device=dev)
    ks = vs = None
    if cdt == "e4m3":
        ks = torch.empty(num_pages, hkv, page_size, dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
    table = torch.zeros(max(B, 1), stride, dtype=torch.int32, device=dev)
    cache = PagedKVCache(kp, vp, table, ks, vs)
    kv_lens = torch.empty(max(B, 0), dtype=torch.int32, device=dev)
    c = cache.struct()
    st = lib().nk_attention_pack(_ptr(k), _ptr(v), _dtype_code(k.dtype), _ptr(key_offsets), _ptr(key_lengths),
                                 ctypes.byref(c), _ptr(kv_lens), B, int(max_key_len), _stream(stream))
    _check(st, "nk_attention_pack")
    return cache, kv_lens, int(max_key_len)


def ragged_paged_attention_backward(q, q_offsets, kv_lens, cache, softmax_scale, max_kv_len, out, dout, lse,
                                    key_offsets, num_key_rows, window_left=-1, window_right=0, sink_keys=0,
                                    dq=None, dk=None, dv=None, stream=None):
    """Gradients (dq [T, Hq, D], dk, dv [num_key_rows, Hkv, D], float32) of
    ragged_paged_attention from its out, lse and the output gradient dout;
    segment s's key j has its dk, dv at row key_offsets[s] + j.  The library
    writes only the rows of kept keys (key_offsets[s] .. + kv_lens[s] - 1);
    when dk/dv are not given they are allocated zero-filled, so rows of keys
    left out of the pack (a key nobody reads has zero gradient) come back as
    zeros; caller-given dk/dv keep their contents in those rows."""
    T, hq, d = q.shape
    B = kv_lens.shape[0]
    _i32(q_offsets, "q_offsets"), _i32(kv_lens, "kv_lens"), _i32(key_offsets, "key_offsets")
    _dev(q, q_offsets, kv_lens, out, dout, lse, key_offsets, cache.k_pages, dq, dk, dv)
    if out.shape != q.shape or dout.shape != q.shape or out.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("out and dout must match q")
    if lse.shape != (T, hq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [T, Hq]")
    f = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(T, hq, d, **f) if dq is None else dq
    dk = torch.zeros(num_key_rows, cache.num_kv_heads, d, **f) if dk is None else dk
    dv = torch.zeros(num_key_rows, cache.num_kv_heads, d, **f) if dv is None else dv
    c = cache.struct()
    st = lib().nk_ragged_paged_attention_backward(
        _ptr(q), _dtype_code(q.dtype), _ptr(q_offsets), _ptr(kv_lens), ctypes.byref(c), float(softmax_scale),
        int(window_left), int(window_right), int(sink_keys), _ptr(out), _ptr(dout), _ptr(lse), _ptr(key_offsets),
        _ptr(dq), _ptr(dk), _ptr(dv), B, T, int(max_kv_len), hq, _stream(stream))
    _check(st, "nk_ragged_paged_attention_backward")
    return dq, dk, dv


PROFILE_FAMILIES = ("rope_write", "attn_decode", "attn_prefill", "attn_f32", "lse_merge", "attention_pack",
                    "attn_backward")


def profile_enable(on=True, families=None):
    """Time the kernels of `families` (default: all) with HIP events attached
    to their dispatches; on=False turns timing off."""
    fams = PROFILE_FAMILIES if families is None else families
    mask = 0
    for f in fams:
        mask |= 1 << PROFILE_FAMILIES.index(f)
    _check(lib().nk_profile_enable(mask if on else 0), "nk_profile_enable")


def profile_reset():
    lib().nk_profile_reset()


def profile_read(kernel):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().nk_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "nk_profile_read")
    return ms.value, n.value
