"""The C-ABI library on the host: it loads without a GPU, exports every
function include/nk.h declares, and rejects invalid arguments with status
codes before anything is launched (no device needed for these paths)."""

import ctypes
import os
import re

import pytest

from ragged_paged_kv_amd import nk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "nk.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|int32_t|const char \*)\s*(nk_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nk.LIB_PATH):
        pytest.skip("libnk.so not built")
    return nk.lib()


def test_exports_every_declared_function(L):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in nk.h but not exported"
    assert set(nk.EXPORTS) == set(names)


def test_status_strings_and_version(L):
    for code, word in ((0, "ok"), (1, "invalid"), (2, "unsupported"), (3, "workspace"), (4, "device")):
        assert word in nk.status_string(code)
    assert "unknown" in nk.status_string(99)
    assert L.nk_version() >= 10000


def _cache(dtype=nk.NK_BF16, head_dim=128, page_size=16, heads=2, ptr=1):
    return nk.nk_paged_kv_t(ptr, ptr, ptr if dtype == nk.NK_E4M3 else None, ptr if dtype == nk.NK_E4M3 else None,
                            dtype, 4, page_size, heads, head_dim, ptr, 4)


def rope(L, cache, **kw):
    a = dict(q=1, k=1, v=1, in_dtype=nk.NK_BF16, q_out=1, q_offsets=1, kv_lens=1, pos=None, freqs=1, max_pos=16,
             rotary_dim=128, layout=0, num_seqs=1, total=4, hq=4)
    a.update(kw)
    c = cache
    return L.nk_rope_qk_write_paged(a["q"], a["k"], a["v"], a["in_dtype"], a["q_out"], a["q_offsets"], a["kv_lens"],
                                    a["pos"], a["freqs"], a["max_pos"], a["rotary_dim"], a["layout"], a["num_seqs"],
                                    a["total"], a["hq"], None if c is None else ctypes.byref(c), None)


def attn(L, cache, **kw):
    a = dict(q=1, q_dtype=nk.NK_BF16, q_offsets=1, kv_lens=1, scale=0.1, window=-1, out=1, lse=None, num_seqs=1,
             total=4, max_q=4, max_kv=64, hq=4, split=0, ws=None, ws_bytes=0)
    a.update(kw)
    return L.nk_ragged_paged_attention(a["q"], a["q_dtype"], a["q_offsets"], a["kv_lens"],
                                       None if cache is None else ctypes.byref(cache), a["scale"], a["window"],
                                       a["out"], a["lse"], a["num_seqs"], a["total"], a["max_q"], a["max_kv"],
                                       a["hq"], a["split"], a["ws"], a["ws_bytes"], None)


def test_rope_validation(L):
    c = _cache()
    assert rope(L, None) == nk.NK_ERR_INVALID_ARG
    assert rope(L, c, q=None) == nk.NK_ERR_INVALID_ARG
    assert rope(L, c, hq=3) == nk.NK_ERR_INVALID_ARG                 # not a multiple of Hkv
    assert rope(L, c, rotary_dim=24) == nk.NK_ERR_UNSUPPORTED        # not a multiple of 16
    assert rope(L, c, rotary_dim=256) == nk.NK_ERR_UNSUPPORTED       # > head_dim
    assert rope(L, c, layout=5) == nk.NK_ERR_INVALID_ARG
    assert rope(L, c, in_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED   # f32 inputs with a bf16 cache
    assert rope(L, _cache(head_dim=96)) == nk.NK_ERR_UNSUPPORTED
    assert rope(L, _cache(page_size=8)) == nk.NK_ERR_UNSUPPORTED
    assert rope(L, c, max_pos=0) == nk.NK_ERR_INVALID_ARG
    assert rope(L, c, total=-1) == nk.NK_ERR_INVALID_ARG
    e = _cache(nk.NK_E4M3)
    e.k_scales = None
    assert rope(L, e) == nk.NK_ERR_INVALID_ARG                       # e4m3 without scales
    assert rope(L, c, total=0) == nk.NK_OK                           # empty batch: nothing launched


def test_attention_validation(L):
    c = _cache()
    assert attn(L, None) == nk.NK_ERR_INVALID_ARG
    assert attn(L, c, out=None) == nk.NK_ERR_INVALID_ARG
    assert attn(L, c, window=-2) == nk.NK_ERR_INVALID_ARG
    assert attn(L, c, split=48) == nk.NK_ERR_INVALID_ARG             # not a multiple of 32
    assert attn(L, c, scale=float("nan")) == nk.NK_ERR_INVALID_ARG
    assert attn(L, c, q_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED
    assert attn(L, c, hq=5) == nk.NK_ERR_INVALID_ARG                 # not a multiple of Hkv
    # decode rows with more than one chunk need the workspace
    need = L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 8, 8, 1, 100000, 4, 2, 128, -1, 512)
    assert need > 0
    assert attn(L, c, num_seqs=8, total=8, max_q=1, max_kv=100000, split=512) == nk.NK_ERR_WORKSPACE
    assert attn(L, c, num_seqs=8, total=8, max_q=1, max_kv=100000, split=512, ws=1, ws_bytes=need - 1) == nk.NK_ERR_WORKSPACE
    assert attn(L, c, total=0) == nk.NK_OK


def attn_band(L, cache, window_right, **kw):
    a = dict(q=1, q_dtype=nk.NK_BF16, q_offsets=1, kv_lens=1, scale=0.1, window=-1, out=1, lse=None, num_seqs=1,
             total=4, min_q=0, max_q=4, max_kv=64, hq=4, split=0, ws=None, ws_bytes=0, sinks=0)
    a.update(kw)
    return L.nk_ragged_paged_attention_band(a["q"], a["q_dtype"], a["q_offsets"], a["kv_lens"],
                                            None if cache is None else ctypes.byref(cache), a["scale"], a["window"],
                                            window_right, a["sinks"], a["out"], a["lse"], a["num_seqs"], a["total"],
                                            a["min_q"], a["max_q"], a["max_kv"], a["hq"], a["split"], a["ws"],
                                            a["ws_bytes"], None)


def test_band_validation(L):
    c = _cache()
    assert attn_band(L, c, -2) == nk.NK_ERR_INVALID_ARG               # only -1 stands for unbounded
    assert attn_band(L, c, 3, window=-2) == nk.NK_ERR_INVALID_ARG
    assert attn_band(L, None, 0) == nk.NK_ERR_INVALID_ARG
    assert attn_band(L, c, 5, q_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED
    assert attn_band(L, c, -1, total=0) == nk.NK_OK                   # empty batch: nothing launched
    assert attn_band(L, c, 0, window=8, sinks=-1) == nk.NK_ERR_INVALID_ARG
    assert attn_band(L, c, 0, window=8, sinks=4, total=0) == nk.NK_OK
    assert attn_band(L, c, 0, min_q=-1) == nk.NK_ERR_INVALID_ARG
    assert attn_band(L, c, 0, min_q=5, max_q=4) == nk.NK_ERR_INVALID_ARG   # above the upper bound


def test_workspace_and_split_queries(L):
    # no workspace when every decode row fits in one chunk, or without decode-capable dtypes
    assert L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 4, 4, 1, 100, 8, 2, 128, -1, 0) == 0
    assert L.nk_ragged_paged_attention_workspace_size(nk.NK_F32, nk.NK_F32, 4, 4, 1, 100000, 8, 2, 128, -1, 0) == 0
    s = L.nk_ragged_paged_attention_split_tokens(32, 4096, 32, 8, 128, -1, 0)
    assert s % 32 == 0 and 128 <= s <= 4096
    assert L.nk_ragged_paged_attention_split_tokens(32, 4096, 32, 8, 128, -1, 512) == 512
    # wider heads move more bytes per key: fewer, longer chunks
    s128 = L.nk_ragged_paged_attention_split_tokens(64, 8192, 16, 8, 128, 1023, 0)
    s256 = L.nk_ragged_paged_attention_split_tokens(64, 8192, 16, 8, 256, 1023, 0)
    assert s256 > s128 and s256 % 32 == 0 and s128 % 32 == 0
    # a window bounds the visible keys, so the chunk count and workspace shrink
    ws_full = L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 8, 8, 1, 100000, 4, 2, 128, -1, 512)
    ws_win = L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 8, 8, 1, 100000, 4, 2, 128, 1023, 512)
    assert 0 < ws_win < ws_full
    # a window whose band fits one chunk still reserves a second chunk per
    # decode row: the sink keys left of the window (none without a window)
    assert L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 8, 8, 1, 100000, 4, 2, 128, 100, 512) > 0
    assert L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 8, 8, 1, 100, 4, 2, 128, 99, 512) == 0


def test_merge_validation(L):
    f = L.nk_attention_lse_merge
    assert f(1, 1, 1, 2, 4, 127, 1, nk.NK_F32, None, None) == nk.NK_ERR_INVALID_ARG   # odd head_dim
    assert f(1, 1, 1, 2, 4, 1024, 1, nk.NK_F32, None, None) == nk.NK_ERR_INVALID_ARG  # too wide
    assert f(1, 1, 1, 2, 4, 128, 1, nk.NK_E4M3, None, None) == nk.NK_ERR_UNSUPPORTED
    assert f(None, 1, 1, 2, 4, 128, 1, nk.NK_F32, None, None) == nk.NK_ERR_INVALID_ARG
    assert f(1, 1, 1, 0, 4, 128, 1, nk.NK_F32, None, None) == nk.NK_OK


def test_profile_api_without_gpu(L):
    assert L.nk_profile_enable(0) == 0
    ms, n = nk.profile_read("attn_decode")
    assert n == 0 and ms == 0.0
    assert L.nk_profile_enable(1 << 7) == nk.NK_ERR_INVALID_ARG       # no such family
    assert L.nk_profile_enable(-1) == nk.NK_ERR_INVALID_ARG
    nk.profile_enable(True, ["attn_decode", "lse_merge"])             # host-side only, no launch
    nk.profile_enable(False)


def test_mrope_validation(L):
    c = _cache()

    def mrope(sections, pos=1, **kw):
        a = dict(q=1, k=1, v=1, in_dtype=nk.NK_BF16, q_out=1, q_offsets=1, kv_lens=1, freqs=1, max_pos=64,
                 rotary_dim=128, layout=nk.NK_ROPE_HALF, num_seqs=1, total=4, hq=4)
        a.update(kw)
        arr = None if sections is None else (ctypes.c_int32 * max(len(sections), 1))(*sections)
        return L.nk_rope_qk_write_paged_mrope(a["q"], a["k"], a["v"], a["in_dtype"], a["q_out"], a["q_offsets"],
                                              a["kv_lens"], pos, 0 if sections is None else len(sections),
                                              None if arr is None else ctypes.cast(arr, ctypes.c_void_p), a["freqs"],
                                              a["max_pos"], a["rotary_dim"], a["layout"], a["num_seqs"], a["total"],
                                              a["hq"], ctypes.byref(c), None)
    assert mrope([16, 24, 24], total=0) == nk.NK_OK                   # valid, empty batch
    assert mrope([16, 24, 16], total=0) == nk.NK_ERR_INVALID_ARG      # 56 pairs, not rotary_dim/2 = 64
    assert mrope([20, 20, 24], total=0) == nk.NK_ERR_UNSUPPORTED      # not multiples of 8 pairs
    assert mrope([16, 16, 16, 8, 8], total=0) == nk.NK_ERR_INVALID_ARG    # more than 4 sections
    assert mrope([64], pos=None, total=0) == nk.NK_ERR_INVALID_ARG    # sections need position streams
    assert mrope(None, total=0) == nk.NK_OK                           # no sections: the plain call


def pack(L, cache, **kw):
    a = dict(k=1, v=1, in_dtype=nk.NK_BF16, offs=1, lens=None, out=1, num_seqs=2, max_len=64)
    a.update(kw)
    return L.nk_attention_pack(a["k"], a["v"], a["in_dtype"], a["offs"], a["lens"],
                               None if cache is None else ctypes.byref(cache), a["out"], a["num_seqs"],
                               a["max_len"], None)


def test_pack_validation(L):
    c = _cache()                                                      # 4 pages of 16, table stride 4
    assert pack(L, c, num_seqs=-1) == nk.NK_ERR_INVALID_ARG
    assert pack(L, c, max_len=-1) == nk.NK_ERR_INVALID_ARG
    assert pack(L, None) == nk.NK_ERR_INVALID_ARG
    assert pack(L, c, max_len=65) == nk.NK_ERR_INVALID_ARG            # the table row holds 4 pages of 16
    assert pack(L, c, offs=None) == nk.NK_ERR_INVALID_ARG
    assert pack(L, c, out=None) == nk.NK_ERR_INVALID_ARG
    assert pack(L, c, k=None) == nk.NK_ERR_INVALID_ARG
    assert pack(L, c, in_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED    # float32 rows into a bf16 cache
    assert pack(L, _cache(dtype=nk.NK_E4M3), in_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED
    assert pack(L, _cache(head_dim=96)) == nk.NK_ERR_UNSUPPORTED
    assert pack(L, c, num_seqs=0) == nk.NK_OK                         # nothing to pack: no launch


def backward(L, cache, **kw):
    a = dict(q=1, q_dtype=nk.NK_BF16, q_offsets=1, kv_lens=1, scale=0.1, wl=-1, wr=0, sinks=0, out=1, dout=1,
             lse=1, key_offsets=1, dq=1, dk=1, dv=1, num_seqs=1, total=4, max_kv=64, hq=4)
    a.update(kw)
    return L.nk_ragged_paged_attention_backward(
        a["q"], a["q_dtype"], a["q_offsets"], a["kv_lens"], None if cache is None else ctypes.byref(cache),
        a["scale"], a["wl"], a["wr"], a["sinks"], a["out"], a["dout"], a["lse"], a["key_offsets"], a["dq"],
        a["dk"], a["dv"], a["num_seqs"], a["total"], a["max_kv"], a["hq"], None)


def test_backward_validation(L):
    c = _cache()
    assert backward(L, c, total=-1) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, wr=-2) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, sinks=-1) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, scale=float("nan")) == nk.NK_ERR_INVALID_ARG
    assert backward(L, None) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, hq=5) == nk.NK_ERR_INVALID_ARG
    assert backward(L, _cache(dtype=nk.NK_E4M3)) == nk.NK_ERR_UNSUPPORTED
    assert backward(L, c, q_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED
    assert backward(L, c, lse=None) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, key_offsets=None) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, dk=None) == nk.NK_ERR_INVALID_ARG
    assert backward(L, c, num_seqs=0, total=0) == nk.NK_OK


def attn_noalloc(L, cache, **kw):
    a = dict(q=1, q_dtype=nk.NK_BF16, q_offsets=1, kv_lens=1, scale=0.1, window=-1, right=0, sinks=0, out=1,
             lse=None, num_seqs=1, total=4, min_q=0, max_q=4, max_kv=64, hq=16, split=0)
    a.update(kw)
    return L.nk_ragged_paged_attention_noalloc(a["q"], a["q_dtype"], a["q_offsets"], a["kv_lens"],
                                               None if cache is None else ctypes.byref(cache), a["scale"],
                                               a["window"], a["right"], a["sinks"], a["out"], a["lse"],
                                               a["num_seqs"], a["total"], a["min_q"], a["max_q"], a["max_kv"],
                                               a["hq"], a["split"], None)


def test_noalloc_validation(L):
    """The allocation-free entry point checks its arguments like the band
    call and rejects, before launching anything, a call whose workspace
    would exceed the static scratch (the long-context decode batch's
    partials: 128 rows x 64 chunks x 64 heads x 128 dims of float32)."""
    c = _cache(heads=8)
    assert attn_noalloc(L, None) == nk.NK_ERR_INVALID_ARG
    assert attn_noalloc(L, c, right=-2) == nk.NK_ERR_INVALID_ARG
    assert attn_noalloc(L, c, q_dtype=nk.NK_F32) == nk.NK_ERR_UNSUPPORTED
    assert attn_noalloc(L, c, total=0) == nk.NK_OK
    big = L.nk_ragged_paged_attention_workspace_size(nk.NK_BF16, nk.NK_BF16, 128, 128, 1, 32768, 64, 8, 128, -1, 512)
    assert big > nk.NOALLOC_SCRATCH_BYTES
    assert attn_noalloc(L, c, num_seqs=128, total=128, max_q=1, max_kv=32768, hq=64,
                        split=512) == nk.NK_ERR_WORKSPACE
