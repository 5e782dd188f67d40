"""GPU test of the ceiling probes (libmoe_probe.so): each does the work it is timed
for. The read and direct-to-LDS read return the exact sum of the buffer's 32-bit
words, the one-pass tile read the sum of each 32 KiB tile, the copy reproduces its
source, and the matrix-core loop the exact sum of its all-ones products."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "libmoe_probe.so"))
    for n in ("moe_probe_read", "moe_probe_dma_read"):
        getattr(L, n).argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.moe_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.moe_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.moe_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return L


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _word_sum(t):
    w = t.view(torch.int32).cpu().numpy().astype(np.uint32).astype(np.uint64)
    return int(w.sum() % (1 << 32))


@pytest.mark.parametrize("nbytes", [32768 * 3, 32768 * 1000 + 0, 64 << 20])
def test_read_probes_sum_every_word(probe, nbytes):
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(nbytes % 1000)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).to(dev)
    want = _word_sum(buf)
    for fn in (probe.moe_probe_read, probe.moe_probe_dma_read):
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        assert fn(_p(buf), nbytes, _p(sink), None) == 0
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().astype(np.uint32)[0]) == want


@pytest.mark.parametrize("nbytes", [16, 32768 * 3 + 48, 60817408])
def test_read_tiles_probe_sums_each_tile(probe, nbytes):
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(nbytes % 997)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).to(dev)
    tiles = -(-nbytes // 32768)
    out = torch.zeros(tiles + 1, dtype=torch.int32, device=dev)
    assert probe.moe_probe_read_tiles(_p(buf), nbytes, _p(out), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.uint32)
    for b in {0, tiles // 2, tiles - 1}:
        assert int(got[b]) == _word_sum(buf[b * 8192:(b + 1) * 8192]), f"tile {b}"
    assert int(got[tiles]) == 0, "wrote past the last tile"
    assert int(got[:tiles].astype(np.uint64).sum() % (1 << 32)) == _word_sum(buf)


def test_copy_probe_copies(probe):
    dev = torch.device("cuda:0")
    src = torch.randn(3 << 20, device=dev)
    dst = torch.zeros_like(src)
    assert probe.moe_probe_copy(_p(src), _p(dst), src.numel() * 4, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_mfma_probe_exact_sum(probe):
    dev = torch.device("cuda:0")
    waves, iters = 64, 1000
    sink = torch.full((waves,), -1.0, device=dev)
    assert probe.moe_probe_mfma(waves, iters, _p(sink), None) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 16 * 32 * iters)
