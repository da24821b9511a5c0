"""The five synthetic workloads and their seeded inputs.

1. ``tiny_prefill_f32``   -- 2 segments (5, 12 tokens), fp32, Hq 4 / Hkv 2,
   D 64, half RoPE theta 1e4, scale 1/8, page size 16, identity pages.
2. ``decode_bf16``        -- 32 decode rows, KV lengths uniform in
   [512, 4096], Hq 32 / Hkv 8, D 128, bf16, half RoPE theta 5e5, page 16,
   permuted pages.
3. ``prefill_bf16``       -- 8 fresh segments, 8192 tokens, Hq 32 / Hkv 8,
   D 128, bf16, half RoPE theta 5e5, explicit positions, page 16.
4. ``mixed_window_bf16``  -- 4 prefill segments of 1024..4096 tokens plus 60
   decode rows of 2048..8192 keys, Hq 16 / Hkv 8, D 256, window 1024,
   scale 1.0 with unit-RMS Q/K, interleaved RoPE on the first 128 dims
   (theta 1e4), page 32, permuted pages.
5. ``decode_fp8``         -- 128 decode rows, KV lengths log-uniform in
   [4096, 32768], Hq 64 / Hkv 8, D 128, bf16 Q, e4m3 cache with a float32
   scale per (token, kv head), half RoPE theta 1e6, page 16, permuted pages,
   512-token KV splits.
"""

import math
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

NAMES = ("tiny_prefill_f32", "decode_bf16", "prefill_bf16", "mixed_window_bf16", "decode_fp8")
# beyond the five: the prefill batch under a band unbounded on both sides
# (every row sees its whole segment), with M-RoPE and with p-RoPE; the mixed
# batch with 4 sink keys beside its window
EXTRA = ("prefill_bidir_bf16", "prefill_mrope_bf16", "prefill_prope_bf16", "mixed_sinks_bf16")


def names():
    return NAMES


@dataclass
class Workload:
    name: str
    seed: int
    q_lens: np.ndarray          # int32 [B]
    kv_lens: np.ndarray         # int32 [B], keys after the append
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rotary_dim: int
    rope_layout: str            # "half" | "interleaved"
    rope_theta: float
    page_size: int
    in_dtype: str               # "f32" | "bf16"
    cache_dtype: str            # "f32" | "bf16" | "e4m3"
    softmax_scale: float
    window_left: int            # -1 = unbounded
    qk_norm: bool
    explicit_positions: bool
    page_table: np.ndarray      # int32 [B, stride]
    num_pages: int
    split_tokens: int           # 0 = library's choice
    seq_ids: np.ndarray = field(default=None)   # original sequence ids (RNG identity)
    token_ids: np.ndarray = field(default=None)  # original token ids
    full_total_q: int = 0       # tokens of the original batch (RNG identity)
    window_right: int = 0       # keys after a row's position it sees: 0 causal, -1 unbounded
    sink_keys: int = 0          # beside a window: the segment's first keys every row also sees
    mrope_sections: tuple = None  # M-RoPE: rotated pairs per section (position streams from mrope_positions)

    @property
    def num_seqs(self):
        return int(len(self.kv_lens))

    @property
    def q_offsets(self):
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def total_q(self):
        return int(np.sum(self.q_lens))

    @property
    def max_q_len(self):
        return int(np.max(self.q_lens)) if len(self.q_lens) else 0

    @property
    def max_kv_len(self):
        return int(np.max(self.kv_lens)) if len(self.kv_lens) else 0

    @property
    def positions(self):
        """Position of every new token: its slot kv_len - q_len + i."""
        out = np.empty(self.total_q, dtype=np.int32)
        offs = self.q_offsets
        for s in range(self.num_seqs):
            n = int(self.q_lens[s])
            out[offs[s]:offs[s] + n] = self.kv_lens[s] - n + np.arange(n)
        return out

    @property
    def position_ids(self):
        """The position ids passed to the fused step, or None."""
        return self.positions if self.explicit_positions else None

    @property
    def max_pos(self):
        return int(self.max_kv_len)

    def subset(self, seqs):
        """The same workload restricted to some sequences, pages renumbered
        compactly in their original order; values are regenerated
        identically (per-sequence / per-token streams)."""
        seqs = np.asarray(seqs, dtype=np.int64)
        offs = self.q_offsets
        tok = np.concatenate([np.arange(offs[s], offs[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, np.int64)
        pt_rows = []
        for s in seqs:
            n = -(-int(self.kv_lens[s]) // self.page_size)
            pt_rows.append(self.page_table[s, :n])
        used = np.unique(np.concatenate(pt_rows)) if pt_rows else np.zeros(0, np.int32)
        remap = {int(p): i for i, p in enumerate(used)}
        stride = max([len(r) for r in pt_rows] + [1])
        pt = np.zeros((len(seqs), stride), dtype=np.int32)
        for i, r in enumerate(pt_rows):
            pt[i, :len(r)] = [remap[int(p)] for p in r]
        return replace(self, q_lens=self.q_lens[seqs].copy(), kv_lens=self.kv_lens[seqs].copy(),
                       page_table=pt, num_pages=len(used),
                       seq_ids=self.seq_ids[seqs].copy(), token_ids=self.token_ids[tok].copy())


def _pages(rng, kv_lens, page_size, order):
    counts = [-(-int(L) // page_size) for L in kv_lens]
    total = sum(counts)
    ids = rng.permutation(total).astype(np.int32) if order == "permuted" else np.arange(total, dtype=np.int32)
    stride = max(counts + [1])
    table = np.zeros((len(kv_lens), stride), dtype=np.int32)
    at = 0
    for s, n in enumerate(counts):
        table[s, :n] = ids[at:at + n]
        at += n
    return table, total


def make(which):
    """Workload by number (1..5) or name."""
    if which == "mixed_sinks_bf16":                    # StreamingLLM: 4 sink keys beside the window
        return replace(make("mixed_window_bf16"), name=which, sink_keys=4)
    if which in EXTRA:
        w = replace(make("prefill_bf16"), name=which)
        if which == "prefill_bidir_bf16":
            w.window_right = -1
        elif which == "prefill_mrope_bf16":            # three position streams over 16/24/24 pairs
            w.mrope_sections = (16, 24, 24)
        else:                                          # p-RoPE, a quarter of the pairs rotated
            w.rope_layout, w.rotary_dim = "half_proportional", w.head_dim // 4
        return w
    k = NAMES.index(which) + 1 if isinstance(which, str) else int(which)
    seed = k - 1
    rng = np.random.default_rng(seed)
    if k == 1:
        q_lens = np.array([5, 12], np.int32)
        kv_lens = q_lens.copy()
        table, npages = _pages(rng, kv_lens, 16, "identity")
        w = Workload("tiny_prefill_f32", seed, q_lens, kv_lens, 4, 2, 64, 64, "half", 1e4, 16,
                     "f32", "f32", 1.0 / 8.0, -1, False, True, table, npages, 0)
    elif k == 2:
        kv_lens = rng.integers(512, 4096, endpoint=True, size=32).astype(np.int32)
        q_lens = np.ones(32, np.int32)
        table, npages = _pages(rng, kv_lens, 16, "permuted")
        w = Workload("decode_bf16", seed, q_lens, kv_lens, 32, 8, 128, 128, "half", 5e5, 16,
                     "bf16", "bf16", 1.0 / math.sqrt(128), -1, False, False, table, npages, 0)
    elif k == 3:
        q_lens = np.array([128, 256, 512, 768, 1024, 1536, 1792, 2176], np.int32)
        kv_lens = q_lens.copy()
        table, npages = _pages(rng, kv_lens, 16, "in_order")
        w = Workload("prefill_bf16", seed, q_lens, kv_lens, 32, 8, 128, 128, "half", 5e5, 16,
                     "bf16", "bf16", 1.0 / math.sqrt(128), -1, False, True, table, npages, 0)
    elif k == 4:
        p_lens = rng.integers(1024, 4096, endpoint=True, size=4)
        d_lens = rng.integers(2048, 8192, endpoint=True, size=60)
        q_lens = np.concatenate([p_lens, np.ones(60, np.int64)]).astype(np.int32)
        kv_lens = np.concatenate([p_lens, d_lens]).astype(np.int32)
        table, npages = _pages(rng, kv_lens, 32, "permuted")
        w = Workload("mixed_window_bf16", seed, q_lens, kv_lens, 16, 8, 256, 128, "interleaved",
                     1e4, 32, "bf16", "bf16", 1.0, 1023, True, True, table, npages, 0)
    elif k == 5:
        kv_lens = np.floor(np.exp(rng.uniform(math.log(4096), math.log(32768), 128))).astype(np.int32)
        q_lens = np.ones(128, np.int32)
        table, npages = _pages(rng, kv_lens, 16, "permuted")
        w = Workload("decode_fp8", seed, q_lens, kv_lens, 64, 8, 128, 128, "half", 1e6, 16,
                     "bf16", "e4m3", 1.0 / math.sqrt(128), -1, False, False, table, npages, 512)
    else:
        raise ValueError(which)
    w.seq_ids = np.arange(w.num_seqs)
    w.token_ids = np.arange(w.total_q)
    w.full_total_q = w.total_q
    return w


# ---------------------------------------------------------------- casting
# torch casts run one at a time: the cache is generated from worker threads,
# and torch is not entered concurrently from them
_TORCH_LOCK = threading.Lock()


def _to_storage(x32, dtype):
    """float32 array -> raw storage array (float32 / uint16 bf16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        with _TORCH_LOCK:
            t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
            return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def _fp8_rows(x32):
    """Rows [..., D] float32 -> (codes uint8 [..., D], scale float32 [...])."""
    with _TORCH_LOCK:
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
        scale = t.abs().amax(dim=-1) / 448.0
        safe = torch.where(scale > 0, scale, torch.ones_like(scale))
        y = torch.clamp(t / safe[..., None], -448.0, 448.0)
        codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
        codes = torch.where(scale[..., None] > 0, codes, torch.zeros_like(codes))
        return codes.numpy().copy(), scale.numpy().astype(np.float32)


def _rms_normalize(x32):
    x = x32.astype(np.float64)
    return (x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))).astype(np.float32)


# ---------------------------------------------------------------- new tokens
def _new_tokens_all(w):
    rng = np.random.default_rng([w.seed, 1])
    T_all = w.full_total_q
    q = rng.standard_normal((T_all, w.num_q_heads, w.head_dim), dtype=np.float32)
    k = rng.standard_normal((T_all, w.num_kv_heads, w.head_dim), dtype=np.float32)
    v = rng.standard_normal((T_all, w.num_kv_heads, w.head_dim), dtype=np.float32)
    return q, k, v


def new_tokens(w):
    """The new tokens' q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D] as raw storage
    arrays of the input dtype (float32 or uint16 bf16 bits)."""
    q, k, v = _new_tokens_all(w)
    q, k, v = q[w.token_ids], k[w.token_ids], v[w.token_ids]
    if w.qk_norm:
        q, k = _rms_normalize(q), _rms_normalize(k)
    return {"q": _to_storage(q, w.in_dtype), "k": _to_storage(k, w.in_dtype),
            "v": _to_storage(v, w.in_dtype)}


def mrope_positions(w):
    """M-RoPE position streams [3, T] int32 in the manner of vision-language
    models: temporal = the token's position, then height and width walking
    a 4-wide grid (all below the token's position + 1, so inside the
    table)."""
    p = w.positions.astype(np.int64)
    return np.stack([p, p // 4, p % 4 + p // 16]).astype(np.int32)


def freqs_table(w, max_pos=None):
    """RoPE table [max_pos, R/2, 2] float32 of (cos, sin) at angle
    pos * theta**(-2i/d) for pair i (the RoPE rotation angle of the Algenta
    page's ``rope_rotation_angle``) with d = rotary_dim, or d = head_dim for
    the proportional layout (aria_kernel ``rope_half_proportional``: the full
    head_dim denominator), computed in float64 and rounded to float32."""
    n = w.max_pos if max_pos is None else max_pos
    half = w.rotary_dim // 2
    denom = w.head_dim if w.rope_layout == "half_proportional" else w.rotary_dim
    inv = w.rope_theta ** (-2.0 * np.arange(half, dtype=np.float64) / denom)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


# ---------------------------------------------------------------- prior cache
def prior_rows(w, s):
    """Prior cache rows of local sequence s (slots 0..kv_len-q_len-1) as raw
    storage: (K [n,Hkv,D], V [n,Hkv,D], k_scale [n,Hkv] | None, v_scale)."""
    n = int(w.kv_lens[s]) - int(w.q_lens[s])
    shape = (max(n, 0), w.num_kv_heads, w.head_dim)
    rng = np.random.default_rng([w.seed, 2, int(w.seq_ids[s])])
    K = rng.standard_normal(shape, dtype=np.float32)
    V = rng.standard_normal(shape, dtype=np.float32)
    if w.qk_norm and n > 0:
        K = _rms_normalize(K)
    if w.cache_dtype == "e4m3":
        kc, ks = _fp8_rows(K)
        vc, vs = _fp8_rows(V)
        return kc, vc, ks, vs
    return _to_storage(K, w.cache_dtype), _to_storage(V, w.cache_dtype), None, None


_SENTINEL = {"f32": (np.float32, np.uint32(0xFFFFFFFF)), "bf16": (np.uint16, np.uint16(0xFFFF)),
             "e4m3": (np.uint8, np.uint8(0xFF))}


# 16-dim groups per 16-byte V run: 4 / element bytes
_V_RUN = {"f32": 1, "bf16": 2, "e4m3": 4}


def sentinel_cache(w):
    """Empty cache storage: every element the dtype's all-ones NaN pattern,
    scales NaN.  Returns dict(k_pages [pages, heads, D/(32 NK), P, 32 NK]
    (NK 2 for e4m3, else 1), v_pages
    [pages, heads, P/16, D/(16 NV), 64, 4 NV], k_scales, v_scales
    [pages, heads, P]); NV = 4 / element bytes."""
    dt, pat = _SENTINEL[w.cache_dtype]
    nv = _V_RUN[w.cache_dtype]
    nk = 2 if w.cache_dtype == "e4m3" else 1
    kshape = (w.num_pages, w.num_kv_heads, w.head_dim // (32 * nk), w.page_size, 32 * nk)
    vshape = (w.num_pages, w.num_kv_heads, w.page_size // 16, w.head_dim // (16 * nv), 64, 4 * nv)
    if w.cache_dtype == "f32":
        k = np.full(kshape, pat, dtype=np.uint32).view(np.float32)
        v = np.full(vshape, pat, dtype=np.uint32).view(np.float32)
    else:
        k = np.full(kshape, pat, dtype=dt)
        v = np.full(vshape, pat, dtype=dt)
    ks = vs = None
    if w.cache_dtype == "e4m3":
        ks = np.full((w.num_pages, w.num_kv_heads, w.page_size), np.nan, np.float32)
        vs = np.full((w.num_pages, w.num_kv_heads, w.page_size), np.nan, np.float32)
    return {"k_pages": k, "v_pages": v, "k_scales": ks, "v_scales": vs}


def build_cache(w, threads=8):
    """The cache as the step finds it: sentinel everywhere, prior rows of
    every sequence in their slots.  Raw storage dict as ``sentinel_cache``."""
    c = sentinel_cache(w)

    def fill(s):
        K, V, ks, vs = prior_rows(w, s)
        n = K.shape[0]
        if n == 0:
            return
        slots = np.arange(n)
        pages = w.page_table[s][slots // w.page_size].astype(np.int64)
        offs = slots % w.page_size
        # K pages hold blocks of 32*NK dims: [page][head][block][slot][32*NK],
        # a slot's row of a block ordered (8-dim group, 32-dim half, dim)
        nk = 2 if w.cache_dtype == "e4m3" else 1
        kb = K.reshape(n, w.num_kv_heads, w.head_dim // (32 * nk), nk, 4, 8).transpose(0, 1, 2, 4, 3, 5)
        c["k_pages"][pages, :, :, offs, :] = kb.reshape(n, w.num_kv_heads, w.head_dim // (32 * nk), 32 * nk)
        # V pages: per 16-slot block, runs 16*g + l of 4 slots x NV dims
        nv = _V_RUN[w.cache_dtype]
        d = np.arange(w.head_dim)
        grp, j, l = (d // 16) // nv, (d // 16) % nv, d % 16
        lane = 16 * ((offs % 16) // 4)[:, None] + l[None, :]
        pos = 4 * j[None, :] + (offs % 4)[:, None]
        heads = np.arange(w.num_kv_heads)
        c["v_pages"][pages[:, None, None], heads[None, :, None], (offs // 16)[:, None, None],
                     grp[None, None, :], lane[:, None, :], pos[:, None, :]] = V
        if ks is not None:
            c["k_scales"][pages, :, offs] = ks
            c["v_scales"][pages, :, offs] = vs

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(w.num_seqs)))
    return c


def custom(q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim, *, rotary_dim=None,
           rope_layout="half", rope_theta=1e4, page_size=16, in_dtype="bf16", cache_dtype="bf16",
           softmax_scale=None, window_left=-1, qk_norm=False, explicit_positions=True,
           page_order="permuted", seed=1000, split_tokens=0, name="custom", window_right=0,
           sink_keys=0):
    """A workload of given shapes (for tests); pages drawn from
    ``default_rng(seed)``, values from the same per-token/per-sequence streams
    as the named workloads."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    table, npages = _pages(rng, kv_lens, page_size, page_order)
    w = Workload(name, seed, q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim,
                 head_dim if rotary_dim is None else rotary_dim, rope_layout, rope_theta, page_size,
                 in_dtype, cache_dtype, 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale,
                 window_left, qk_norm, explicit_positions, table, npages, split_tokens)
    w.seq_ids = np.arange(w.num_seqs)
    w.token_ids = np.arange(w.total_q)
    w.full_total_q = w.total_q
    w.window_right = window_right
    w.sink_keys = sink_keys
    return w
