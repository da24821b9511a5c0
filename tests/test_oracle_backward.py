"""Pins of the oracle's attention gradients (NumKong matrix-kernels page,
attention_packed_gradients): the closed-form softmax-Jacobian gradients
against torch autograd through a float64 CPU forward written with an explicit
mask (an independent differentiation of the same forward), under causal,
windowed, two-sided and sink bands with GQA; and a central finite difference
of the oracle's own forward on a tiny case."""

import numpy as np
import pytest
import torch

from oracle import attention as o_attn
from oracle.paged import PagedCache


def _setup(rng, q_lens, kv_lens, hq, hkv, d, P=16):
    npages = sum(-(-L // P) for L in kv_lens)
    cache = PagedCache("f32", npages, hkv, P, d)
    stride = max(-(-L // P) for L in kv_lens)
    table = np.zeros((len(kv_lens), stride), dtype=np.int64)
    perm = rng.permutation(npages)
    at = 0
    Ks, Vs = [], []
    for s, L in enumerate(kv_lens):
        n = -(-L // P)
        table[s, :n] = perm[at:at + n]
        at += n
        K = rng.standard_normal((L, hkv, d))
        V = rng.standard_normal((L, hkv, d))
        for j in range(L):
            for h in range(hkv):
                cache.store(table, s, j, h, K[j, h], V[j, h])
        Ks.append(K)
        Vs.append(V)
    T = sum(q_lens)
    q = rng.standard_normal((T, hq, d))
    dout = rng.standard_normal((T, hq, d))
    q_offsets = np.concatenate([[0], np.cumsum(q_lens)])
    return cache, table, Ks, Vs, q, dout, q_offsets


def _torch_grads(q, dout, Ks, Vs, q_offsets, kv_lens, scale, wl, wr, sinks, hq, hkv):
    group = hq // hkv
    qt = torch.tensor(q, requires_grad=True)
    kts = [torch.tensor(K, requires_grad=True) for K in Ks]
    vts = [torch.tensor(V, requires_grad=True) for V in Vs]
    outs = []
    for s, L in enumerate(kv_lens):
        a, b = int(q_offsets[s]), int(q_offsets[s + 1])
        ql = b - a
        p = torch.arange(ql)[:, None] + L - ql
        k = torch.arange(L)[None, :]
        hi = torch.full_like(p, L - 1) if wr < 0 else torch.clamp(p + wr, max=L - 1)
        lo = torch.zeros_like(p) if wl < 0 else torch.clamp(p - wl, min=0)
        vis = (k <= hi) & ((k >= lo) | (k < sinks))
        for h in range(hq):
            g = h // group
            sc = scale * qt[a:b, h] @ kts[s][:, g].T
            sc = torch.where(vis, sc, torch.tensor(-torch.inf, dtype=torch.float64))
            w = torch.softmax(sc, dim=-1)
            w = torch.where(vis.any(dim=-1, keepdim=True), w, torch.zeros_like(w))
            outs.append((w @ vts[s][:, g], a, b, h))
    loss = sum((o * torch.tensor(dout[a:b, h])).sum() for o, a, b, h in outs)
    loss.backward()
    return qt.grad.numpy(), [t.grad.numpy() for t in kts], [t.grad.numpy() for t in vts]


@pytest.mark.parametrize("band", [(-1, 0, 0), (5, 0, 0), (4, 3, 0), (6, 0, 3), (-1, -1, 0)])
def test_backward_against_autograd(band):
    wl, wr, sinks = band
    rng = np.random.default_rng(11)
    q_lens, kv_lens, hq, hkv, d = [4, 1, 9, 12], [4, 20, 30, 9], 4, 2, 32
    cache, table, Ks, Vs, q, dout, q_offsets = _setup(rng, q_lens, kv_lens, hq, hkv, d)
    dq, dk, dv = o_attn.ragged_paged_attention_backward(q, q_offsets, kv_lens, cache, table, 0.2, dout,
                                                        wl, wr, sinks)
    tq, tk, tv = _torch_grads(q, dout, Ks, Vs, q_offsets, kv_lens, 0.2, wl, wr, sinks, hq, hkv)
    assert np.allclose(dq, tq, rtol=0, atol=1e-12)
    for s in range(len(kv_lens)):
        assert np.allclose(dk[s], tk[s], rtol=0, atol=1e-12)
        assert np.allclose(dv[s], tv[s], rtol=0, atol=1e-12)


def test_backward_finite_difference():
    rng = np.random.default_rng(12)
    q_lens, kv_lens, hq, hkv, d = [3, 1], [5, 7], 2, 1, 16
    cache, table, Ks, Vs, q, dout, q_offsets = _setup(rng, q_lens, kv_lens, hq, hkv, d)
    dq, dk, dv = o_attn.ragged_paged_attention_backward(q, q_offsets, kv_lens, cache, table, 0.3, dout, 2, 0, 1)

    def loss(qq, cc):
        out, _ = o_attn.ragged_paged_attention(qq, q_offsets, kv_lens, cc, table, 0.3, 2, window_right=0,
                                               sink_keys=1)
        return float(np.sum(out * dout))

    eps = 1e-6
    for (t, h, i) in [(0, 0, 3), (2, 1, 7), (3, 0, 0)]:
        qp, qm = q.copy(), q.copy()
        qp[t, h, i] += eps
        qm[t, h, i] -= eps
        assert abs((loss(qp, cache) - loss(qm, cache)) / (2 * eps) - dq[t, h, i]) < 1e-7
    for (s, j, i) in [(0, 4, 2), (1, 0, 5), (1, 6, 9)]:
        for which, grad in (("k", dk), ("v", dv)):
            cp, cm = cache.copy(), cache.copy()
            page, off = cp.locate(table, s, j)
            arr_p = cp.k if which == "k" else cp.v
            arr_m = cm.k if which == "k" else cm.v
            if which == "k":
                arr_p[page, 0, off, i] += eps
                arr_m[page, 0, off, i] -= eps
            else:
                arr_p[page, 0, i, off] += eps
                arr_m[page, 0, i, off] -= eps
            fd = (loss(q, cp) - loss(q, cm)) / (2 * eps)
            assert abs(fd - grad[s][j, 0, i]) < 1e-7, (which, s, j, i)
