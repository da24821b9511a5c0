"""Ragged paged attention with fused RoPE + KV append for AMD MI355X (gfx950).

The compute path is the HIP library ``libnk.so`` (C ABI in ``include/nk.h``);
``ragged_paged_kv_amd.nk`` is its thin ctypes binding.
"""

from .nk import (PagedKVCache, rope_qk_write_paged, ragged_paged_attention,  # noqa: F401
                 attention_lse_merge, workspace_size, split_tokens, NKError, lib)
