"""Float64 CPU oracle for ragged paged attention with fused RoPE + KV append.

TEST INFRASTRUCTURE ONLY.  This package is the independent reference that the
HIP path is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path (the
``ragged_paged_kv_amd`` package and its C-ABI library) never does, and this
package imports nothing from it.

Everything here is plain numpy in float64, written from the definitions on the
source pages, with no blocking, fusion or reordering beyond what those
definitions state:

* ``formats``   -- bfloat16 and float8 e4m3fn encode/decode (round to nearest,
                   ties to even; e4m3 saturating), per the NumKong Python page,
                   "Scalar Types" table and "Buffer-First Casting".
* ``paged``     -- the paged cache layout of ``include/nk.h`` read and written
                   element by element.
* ``rope``      -- rotary embedding of Q and K from a (cos, sin) table and the
                   append of K/V into cache pages (Mojo page,
                   ``generic_fused_qk_rope_bshd_paged_ragged_kernel_api``;
                   NumKong matrix-kernels page, ``attention_rope``; aria_kernel
                   crate, ``rope`` / ``rope_half`` / ``rope_half_partial``).
* ``pack``      -- ragged K/V token rows packed into the paged cache (NumKong
                   matrix-kernels page, ``attention_pack``).
* ``attention`` -- ragged scaled-dot-product attention under a key band
                   (NumKong matrix-kernels page, "Attention with a Pre-Packed
                   KV-Cache" and ``attention_packed``; Algenta "Attention
                   variant kernels", "A scalar reference, not a buffer kernel").
* ``merge``     -- log-sum-exp merge of partial attention states (Algenta,
                   "Flash attention's running state reproduces the same
                   softmax").
* ``brute``     -- pure-Python loops (``math.exp``/``math.fsum``) of the same
                   definitions for tiny inputs.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants, library routines or brute force.
"""

from . import formats, paged, pack, rope, attention, merge, brute  # noqa: F401
