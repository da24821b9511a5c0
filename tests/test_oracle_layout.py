"""Pins of the oracle's cache storage conversion: the V page order equals the
offset formula stated in include/nk.h element by element, and storage ->
values -> storage is the identity (K and V, every element type)."""

import numpy as np
import pytest

from oracle.paged import (PagedCache, k_logical_to_storage, k_storage_to_logical, v_logical_to_storage,
                          v_storage_to_logical)


def _formula(d, t, D, nv):
    c = (d // 16) // nv
    return ((t // 16) * (D // (16 * nv)) + c) * 64 * 4 * nv + (16 * ((t % 16) // 4) + d % 16) * 4 * nv \
        + ((d // 16) % nv) * 4 + t % 4


@pytest.mark.parametrize("dtype,nv", [("f32", 1), ("bf16", 2), ("e4m3", 4)])
@pytest.mark.parametrize("D,P", [(64, 16), (128, 32), (256, 16)])
def test_v_order_is_the_header_formula(dtype, nv, D, P):
    rng = np.random.default_rng(7)
    logical = rng.integers(0, 1 << 16, size=(3, 2, D, P))
    raw = v_logical_to_storage(dtype, logical)
    assert raw.shape == (3, 2, P // 16, D // (16 * nv), 64, 4 * nv)
    flat = raw.reshape(3, 2, -1)
    for d in range(0, D, 7):
        for t in range(P):
            assert flat[1, 1, _formula(d, t, D, nv)] == logical[1, 1, d, t]
    np.testing.assert_array_equal(v_storage_to_logical(dtype, raw), logical)


@pytest.mark.parametrize("dtype,nk", [("f32", 1), ("bf16", 1), ("e4m3", 2)])
@pytest.mark.parametrize("D,P", [(64, 16), (128, 32), (256, 16)])
def test_k_order_is_the_header_formula(dtype, nk, D, P):
    rng = np.random.default_rng(9)
    logical = rng.integers(0, 1 << 16, size=(3, 2, P, D))          # [page][head][token][dim]
    raw = k_logical_to_storage(dtype, logical)
    assert raw.shape == (3, 2, D // (32 * nk), P, 32 * nk)
    flat = raw.reshape(3, 2, -1)
    for d in range(0, D, 5):
        for t in range(P):
            idx = ((d // (32 * nk)) * P + t) * 32 * nk + ((d % 32) // 8) * nk * 8 + ((d // 32) % nk) * 8 + d % 8
            assert flat[0, 1, idx] == logical[0, 1, t, d]
    np.testing.assert_array_equal(k_storage_to_logical(dtype, raw), logical)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_storage_round_trip(dtype):
    rng = np.random.default_rng(8)
    n, h, p, d = 5, 2, 32, 128
    if dtype == "f32":
        k = rng.standard_normal((n, h, d // 32, p, 32)).astype(np.float32)
        v = rng.standard_normal((n, h, p // 16, d // 16, 64, 4)).astype(np.float32)
    elif dtype == "bf16":
        k = rng.integers(0, 0x7f80, size=(n, h, d // 32, p, 32)).astype(np.uint16)
        v = rng.integers(0, 0x7f80, size=(n, h, p // 16, d // 32, 64, 8)).astype(np.uint16)
    else:
        k = rng.integers(0, 0x7f, size=(n, h, d // 64, p, 64)).astype(np.uint8)
        v = rng.integers(0, 0x7f, size=(n, h, p // 16, d // 64, 64, 16)).astype(np.uint8)
    ks = vs = None
    if dtype == "e4m3":
        ks = rng.random((n, h, p)).astype(np.float32)
        vs = rng.random((n, h, p)).astype(np.float32)
    c = PagedCache.from_storage(dtype, k, v, ks, vs)
    k2, v2, ks2, vs2 = c.to_storage()
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
    if dtype == "e4m3":
        np.testing.assert_array_equal(ks2, ks)
        np.testing.assert_array_equal(vs2, vs)
