"""GPU tests of the packed weight layout, the library's weight format for bf16
matrices: moe_pack_weights moves every element to the place include/moe.h
states (bit for bit; expert tensors and single projection matrices), and the
Python binding refuses a weight tensor that was never packed. That the layer on
packed weights computes the right thing is the parity tests' business (they
pack the row-major weights the oracle reads)."""
import pytest
import torch

from synthetic import make_inputs, scaled_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_fp32_amd  # noqa: F401  (fails loudly if libmoe.so is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def moe(dev):
    import sparse_mixture_experts_fp32_amd as m
    return m


def _unpack(p):
    """Packed [G, N, K] -> row-major: tile (n // 16, k // 32) is 512 contiguous elements,
    element (r, c) of it at (r + 16 * (c // 8)) * 8 + c % 8."""
    G, N, K = p.shape
    t = p.reshape(G, N // 16, K // 32, 4, 16, 8)  # (.., column group c // 8, row r, c % 8)
    return t.permute(0, 1, 4, 2, 3, 5).reshape(G, N, K)


@pytest.mark.parametrize("G,N,K", [(3, 32, 128), (2, 48, 96), (1, 2048, 7168), (0, 16, 32)])
def test_pack_weights_layout(dev, moe, G, N, K):
    g = torch.Generator(device="cpu").manual_seed(G * N + K)
    w = torch.randn((G, N, K), generator=g).to(torch.bfloat16).to(dev)
    p = moe.moe_pack_weights(w)
    torch.cuda.synchronize()
    assert p.moe_packed and p.shape == w.shape
    assert torch.equal(_unpack(p.view(torch.int16)).view(torch.bfloat16), w)


@pytest.mark.parametrize("N,K", [(384, 256), (7168, 3584)])
def test_pack_single_matrix(dev, moe, N, K):
    """A projection matrix [N, K] packs as one group."""
    g = torch.Generator(device="cpu").manual_seed(N + K)
    w = torch.randn((N, K), generator=g).to(torch.bfloat16).to(dev)
    p = moe.moe_pack_weights(w)
    torch.cuda.synchronize()
    assert p.moe_packed and p.shape == w.shape
    assert torch.equal(_unpack(p.view(torch.int16).unsqueeze(0)).view(torch.bfloat16)[0], w)


def test_layer_calls_refuse_unpacked_weights(dev, moe):
    cfg = scaled_config("tiny", name="unpacked")
    di = make_inputs(cfg).to(dev)
    fwd = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    with pytest.raises(TypeError, match="packed"):
        fwd(di.x, di.w_router, di.router_bias, di.w_gate, di.w_up, di.w_down)
    pg, pu = moe.moe_pack_weights(di.w_gate), moe.moe_pack_weights(di.w_up)
    with pytest.raises(TypeError, match="w_down"):
        fwd(di.x, di.w_router, di.router_bias, pg, pu, di.w_down)
