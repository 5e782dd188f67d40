"""The packed expert-weight layout of include/moe.h, on the host: the index map
written there (tile (n // 16, k // 32) of 512 elements, element (r, c) of a tile at
(r + 16 * (c // 8)) * 8 + c % 8) is a bijection, and the reshape that the GPU tests
use to unpack (tests/test_gpu_packed.py) inverts exactly that map."""
import numpy as np
import pytest


def _pack_by_formula(w):
    G, N, K = w.shape
    out = np.empty(G * N * K, dtype=w.dtype)
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    dst = ((n // 16) * (K // 32) + k // 32) * 512 + ((n % 16) + 16 * ((k % 32) // 8)) * 8 + k % 8
    for g in range(G):
        out[g * N * K + dst] = w[g]
    return out.reshape(G, N, K)


def _unpack(p):  # as in tests/test_gpu_packed.py, on numpy arrays
    G, N, K = p.shape
    return p.reshape(G, N // 16, K // 32, 4, 16, 8).transpose(0, 1, 4, 2, 3, 5).reshape(G, N, K)


@pytest.mark.parametrize("G,N,K", [(1, 16, 32), (2, 48, 96), (3, 32, 256)])
def test_formula_is_a_bijection_and_unpack_inverts_it(G, N, K):
    w = np.arange(G * N * K, dtype=np.int64).reshape(G, N, K)
    p = _pack_by_formula(w)
    assert np.array_equal(np.sort(p.ravel()), np.arange(G * N * K))  # every element exactly once
    assert np.array_equal(_unpack(p), w)


def test_one_tile_is_one_mfma_operand():
    """Lane l of a 64-lane operand (row l % 16, columns 8 (l // 16) .. + 7) reads the
    16 bytes at 16 l of the tile: the tile is the operand in lane order."""
    w = np.arange(16 * 32, dtype=np.int64).reshape(1, 16, 32)
    tile = _pack_by_formula(w).ravel()
    for lane in range(64):
        r, c0 = lane % 16, 8 * (lane // 16)
        assert np.array_equal(tile[8 * lane:8 * lane + 8], w[0, r, c0:c0 + 8])
