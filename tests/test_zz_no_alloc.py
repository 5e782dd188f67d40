"""GPU test of moe_permute_noalloc, the permute entry point that allocates nothing
(its per-expert, per-chunk counts live in a fixed array inside the library).

Through the C ABI, two calls in a row on one stream -- the first with the
largest count matrix any shape has (1024 experts over 32 chunks), the second
smaller, so it runs over what the first left in the array -- each equal bit for
bit to moe_permute with a caller-owned workspace (offsets, row_of, row_src and
the gathered rows), and to the oracle's permutation.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle.moe_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_mixture_experts_fp32_amd import _lib
    return _lib


def _inputs(T, d, E, k, seed, dev):
    g = torch.Generator().manual_seed(seed)
    idx = torch.argsort(torch.rand((T, E), generator=g), dim=1)[:, :k].to(torch.int32).contiguous()
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    return x.to(dev), idx.to(dev)


def _outputs(T, d, E, k, dev):
    return (torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            torch.full((T, k), -7, dtype=torch.int32, device=dev),
            torch.full((T * k,), -7, dtype=torch.int32, device=dev),
            torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


CALLS = [(4096, 256, 1024, 16, 1), (300, 128, 64, 4, 2)]  # T, d, E, k, seed: the second is smaller


def test_noalloc_permute_two_calls_match_moe_permute(lib):
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    runs = []
    for T, d, E, k, seed in CALLS:
        print(f"noalloc permute: T={T} d={d} E={E} k={k}", flush=True)
        x, idx = _inputs(T, d, E, k, seed, dev)
        s = lib.shape(T, d, E, k, 128)
        got = _outputs(T, d, E, k, dev)
        st = lib.lib.moe_permute_noalloc(ctypes.byref(s), _ptr(x), _ptr(idx), *(_ptr(t) for t in got), stream)
        assert st == lib.MOE_OK, lib.lib.moe_last_error()
        runs.append((T, d, E, k, x, idx, s, got))
    torch.cuda.synchronize()
    for T, d, E, k, x, idx, s, got in runs:
        ref = _outputs(T, d, E, k, dev)
        need = lib.lib.moe_workspace_bytes(ctypes.byref(s), lib.MOE_CALL_PERMUTE)
        assert 0 < need <= 131072
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        st = lib.lib.moe_permute(ctypes.byref(s), _ptr(x), _ptr(idx), *(_ptr(t) for t in ref), _ptr(ws), need,
                                 stream)
        assert st == lib.MOE_OK, lib.lib.moe_last_error()
        torch.cuda.synchronize()
        for name, a, b in zip(("expert_offsets", "row_of", "row_src", "x_perm"), got, ref):
            assert torch.equal(a, b), f"{name} differs from moe_permute (T={T}, E={E})"
        off, row_of, row_src = orc.permute(idx.cpu().numpy(), E)
        assert np.array_equal(got[0].cpu().numpy(), off)
        assert np.array_equal(got[1].cpu().numpy(), row_of)
        assert np.array_equal(got[2].cpu().numpy(), row_src)
        assert torch.equal(got[3].cpu(), x.cpu()[torch.from_numpy(row_src).long()])
