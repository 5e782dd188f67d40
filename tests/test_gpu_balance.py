"""GPU parity of the load-balancing calls (aux loss, Quantile Balancing) against
the CPU oracle, through the C ABI.

Tolerances:
  * integers -- QB ids, histogram counts -- and the float32 values the
    selection itself produces (the cutoff alpha): bit for bit;
  * QB bias: bit for bit (both sides evaluate the same float64 expression,
    operation by operation, on the same integer counts, then round once);
  * QB weights: |dw| <= 1e-5 (same device logits on both sides);
  * expert mean probabilities: |dm_e| <= 1e-5 m_e. Each device probability is
    expf, a float32 sum of at most 16 * 64 exponentials, one reciprocal of that
    sum and one fused multiply-add into the running sum (relative error below
    2e-6); the float32 partial sums over 16 tokens and 4 wavefronts add below
    2e-6 more (all terms positive); float64 after that;
  * aux loss: it moves by sum_e (2 |m_e - 1/E| d_e + d_e^2) for errors d_e of
    the means, plus its own float32 rounding, so
    |dL| <= sum_e (2 |m_e - 1/E| d_e + d_e^2) + 2^-23 L with d_e = 1e-5 m_e.
"""
import numpy as np
import pytest
import torch

import oracle.balance as bal
import oracle.moe_oracle as orc
from tests import gpu_util as gu

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


def _logits(T, E, seed, scale=1.0, zipf=False):
    r = np.random.default_rng(seed)
    L = r.standard_normal((T, E)) * scale
    if zipf:  # the skewed workload's bias: -1.5 ln(rank), ranks a seeded permutation
        L = L + (-1.5 * np.log(r.permutation(E) + 1.0))[None, :]
    return L.astype(np.float32)


def _check_aux(moe, dev, L):
    Lg = torch.from_numpy(L).to(dev)
    pm, aux = moe.moe_aux_loss(Lg)
    torch.cuda.synchronize()
    loss_ref, m_ref = bal.aux_loss(orc.softmax(gu.f64(Lg)))
    m = gu.f64(pm)
    d = 1e-5 * m_ref
    err = np.abs(m - m_ref)
    assert np.all(err <= d + 1e-30), f"prob_mean off by {err.max():.3e} (bound {d.max():.3e})"
    E = L.shape[1]
    bound = np.sum(2 * np.abs(m_ref - 1.0 / E) * d + d * d) + 2.0 ** -23 * loss_ref + 1e-30
    got = float(gu.f64(aux)[0])
    assert abs(got - loss_ref) <= bound, f"aux loss {got} vs {loss_ref} (bound {bound:.3e})"
    return pm, aux


# ---------------------------------------------------------------- aux loss

@pytest.mark.parametrize("T,E", [(64, 8), (1, 5), (130, 96), (1000, 256), (257, 1024), (4099, 896), (65, 63)])
def test_aux_loss_matches_oracle(dev, moe, T, E):
    _check_aux(moe, dev, _logits(T, E, seed=T + 7 * E, scale=2.0))


def test_aux_loss_special_cases(dev, moe):
    """Equal logits: means 1/E and loss ~0; every token sure of expert 3: loss (E-1)/E;
    token t peaked on expert t mod E over whole cycles: means 1/E, loss ~0."""
    E = 40
    pm, aux = _check_aux(moe, dev, np.full((200, E), 0.25, np.float32))
    assert abs(float(aux[0])) < 1e-12
    L = np.full((77, E), -200.0, np.float32)
    L[:, 3] = 200.0
    pm, aux = _check_aux(moe, dev, L)
    assert abs(float(aux[0]) - (E - 1) / E) < 1e-6
    L = np.zeros((3 * E, E), np.float32)
    L[np.arange(3 * E), np.arange(3 * E) % E] = 4.0
    pm, aux = _check_aux(moe, dev, L)
    assert abs(float(aux[0])) < 1e-10


def test_aux_loss_deterministic_and_zero_tokens(dev, moe):
    L = torch.from_numpy(_logits(3000, 384, seed=5)).to(dev)
    a = [t.clone() for t in moe.moe_aux_loss(L)]
    b = moe.moe_aux_loss(L)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(ValueError):
        moe.moe_aux_loss(torch.empty((0, 8), dtype=torch.float32, device=dev))


# ------------------------------------------------------------ QB selection

def _check_qb_route(moe, dev, L, b, k):
    Lg, bg = torch.from_numpy(L).to(dev), torch.from_numpy(b).to(dev)
    idx, w, alpha = moe.moe_qb_route(Lg, bg, k)
    torch.cuda.synchronize()
    idx_ref, alpha_ref = bal.qb_select(L, b, k)
    gi = gu.host(idx).to(torch.int64).numpy()
    mism = np.argwhere(gi != idx_ref)
    assert mism.size == 0, f"QB ids differ at {mism[:5].tolist()} (of {len(mism)})"
    ga = gu.host(alpha).numpy()
    assert np.array_equal(ga, alpha_ref), f"alpha differs at {np.argwhere(ga != alpha_ref)[:5].tolist()}"
    err = np.abs(gu.f64(w) - bal.qb_weights(L, idx_ref))
    assert err.max() <= 1e-5, f"QB weights off by {err.max():.3e}"
    return idx, w, alpha


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (37, 8, 7), (130, 100, 7), (33, 256, 4), (9, 896, 16),
                                   (5, 1024, 63), (70, 64, 63), (1, 2, 1)])
def test_qb_route_matches_oracle(dev, moe, T, E, k):
    L = _logits(T, E, seed=3 * T + E, scale=1.5)
    b = (np.random.default_rng(E).standard_normal(E) * 0.8).astype(np.float32)
    _check_qb_route(moe, dev, L, b, k)


def test_qb_route_ties_and_zero_bias(dev, moe):
    """Integer logits and biases make many exact ties of the biased score (lower id
    wins, -0.0 ties +0.0); with zero bias the ids and weights are the plain top-k's."""
    r = np.random.default_rng(11)
    T, E, k = 90, 72, 6
    L = r.integers(-3, 4, size=(T, E)).astype(np.float32)
    L[0] = 0.0
    L[1, ::2] = -0.0
    b = r.integers(-1, 2, size=E).astype(np.float32)
    b[::5] = -0.0
    _check_qb_route(moe, dev, L, b, k)
    L = _logits(T, E, seed=12)
    idx, w, _ = _check_qb_route(moe, dev, L, np.zeros(E, np.float32), k)
    idx0, w0 = moe.moe_topk_softmax(torch.from_numpy(L).to(dev), k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0)
    assert (w - w0).abs().max().item() <= 1e-6


# ------------------------------------------------------------ QB histogram

def _check_hist(moe, dev, L, alpha, k, lo, width, nb):
    hist = moe.moe_qb_histogram(torch.from_numpy(L).to(dev), torch.from_numpy(alpha).to(dev), k, lo, width, nb)
    torch.cuda.synchronize()
    ref = bal.qb_histogram(L, alpha, lo, width, nb)
    got = gu.host(hist).to(torch.int64).numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"histogram differs at {bad[:5].tolist()} (of {len(bad)})"
    assert np.all(got.sum(axis=1) == L.shape[0])
    return hist


@pytest.mark.parametrize("T,E,k,lo,width,nb", [
    (64, 8, 2, -8.0, 0.015625, 1000),       # 32 experts per block, one ragged slab
    (1000, 96, 7, -12.0, 0.0078125, 1000),  # ragged slab, several token splits
    (333, 100, 4, -6.0, 0.005, 2000),       # 16 experts per block
    (200, 40, 3, -5.0, 0.0025, 4096),       # 8 experts per block
    (129, 33, 2, -1.0, 0.25, 1),            # one bin: every margin counts there
    (70, 896, 16, -8.0, 0.016, 1000),       # the many-expert width
])
def test_qb_histogram_matches_oracle(dev, moe, T, E, k, lo, width, nb):
    L = _logits(T, E, seed=T + E + nb, scale=1.5)
    _, alpha = bal.qb_select(L, np.zeros(E, np.float32), k)
    _check_hist(moe, dev, L, alpha, k, lo, width, nb)


def test_qb_histogram_edges_and_clamping(dev, moe):
    """Margins exactly on bin edges open their bin; margins far outside the range
    clamp to the end bins; T = 0 gives an all-zero histogram."""
    lo, width, nb = -4.0, 0.25, 32
    E, T = 5, 4 * nb
    L = np.zeros((T, E), np.float32)
    for t in range(T):
        L[t] = lo + (t % nb) * width + np.array([0.0, -width / 1024, width / 2, 1e6, -1e6], np.float32)
    alpha = np.zeros(T, np.float32)
    hist = _check_hist(moe, dev, L, alpha, 2, lo, width, nb)
    h = gu.host(hist).numpy()
    assert np.all(h[0] == 4)                          # on the edge: its own bin, 4 rounds
    assert h[1, 0] == 8 and np.all(h[1, 1:nb - 1] == 4) and h[1, nb - 1] == 0  # just below: the bin before
    assert np.all(h[2] == 4)                          # mid-bin
    assert h[3, nb - 1] == T and h[4, 0] == T         # far outside: clamped
    z = moe.moe_qb_histogram(torch.zeros((0, E), dtype=torch.float32, device=dev),
                             torch.zeros(0, dtype=torch.float32, device=dev), 2, lo, width, nb,
                             out=torch.full((E, nb), 7, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert int(z.abs().sum()) == 0


# -------------------------------------------------------------- QB update

@pytest.mark.parametrize("E,k,nb,lo,width", [(8, 2, 1000, -8.0, 0.015625), (96, 7, 64, -3.0, 0.125),
                                             (896, 16, 1000, -8.0, 0.016), (1024, 63, 4096, -5.0, 0.0025),
                                             (3, 1, 1, 0.0, 1.0)])
def test_qb_update_matches_oracle(dev, moe, E, k, nb, lo, width):
    r = np.random.default_rng(E + nb)
    H = r.integers(0, 50, size=(E, nb)) * (r.random((E, nb)) < 0.3)
    H[0] = 0                      # empty row keeps its bias
    if E > 2:
        H[1] = 0
        H[1, nb // 2] = 9         # one occupied bin
        H[2] = 0
        H[2, 0] = 5               # everything in the first bin
    b_in = r.standard_normal(E).astype(np.float32)
    Hg = torch.from_numpy(H.astype(np.int32)).to(dev)
    bg = torch.from_numpy(b_in).to(dev)
    out = moe.moe_qb_update(Hg, k, lo, width, bg)
    torch.cuda.synchronize()
    ref = bal.qb_update(H, k, lo, width, b_in)
    got = gu.host(out).numpy()
    assert np.array_equal(got, ref), f"bias differs at {np.argwhere(got != ref)[:5].tolist()}"
    assert got[0] == b_in[0]
    moe.moe_qb_update(Hg, k, lo, width, bg, out=bg)  # in place
    torch.cuda.synchronize()
    assert np.array_equal(gu.host(bg).numpy(), ref)


# --------------------------------------------------------- QB, whole loop

def test_qb_loop_balances_skewed_router(dev, moe):
    """Route, histogram, update, repeated on one skewed batch, every step checked
    against the oracle on the device's own inputs; the loads end near T k / E."""
    T, E, k = 8192, 64, 4
    lo, width, nb = -16.0, 0.03125, 1000
    L = _logits(T, E, seed=21, zipf=True)
    Lg = torch.from_numpy(L).to(dev)
    bias = torch.zeros(E, dtype=torch.float32, device=dev)
    target = T * k / E
    loads = []
    for _ in range(8):
        b_host = gu.host(bias).numpy().copy()
        idx, w, alpha = _check_qb_route(moe, dev, L, b_host, k)
        loads.append(np.bincount(gu.host(idx).numpy().ravel(), minlength=E) / target)
        hist = moe.moe_qb_histogram(Lg, alpha, k, lo, width, nb)
        new = moe.moe_qb_update(hist, k, lo, width, bias)
        torch.cuda.synchronize()
        H_ref = bal.qb_histogram(L, gu.host(alpha).numpy(), lo, width, nb)
        assert np.array_equal(gu.host(hist).to(torch.int64).numpy(), H_ref)
        assert np.array_equal(gu.host(new).numpy(), bal.qb_update(H_ref, k, lo, width, b_host))
        bias = new
    assert loads[0].max() > 5.0, loads[0].max()
    assert loads[-1].max() < 1.1 and loads[-1].min() > 0.9, (loads[-1].min(), loads[-1].max())


# ------------------------------------------------------------ full size

@pytest.mark.parametrize("zipf", [False, True], ids=["many_expert", "skewed"])
def test_balance_full_size(dev, moe, zipf):
    """The many-expert layer's router outputs (T = 16384, E = 896, k = 16) with
    B = 1000 bins, as the QB step runs them: route, histogram and update bit for
    bit, and the aux loss within its bound."""
    T, E, k = 16384, 896, 16
    lo, width, nb = -16.0, 0.03125, 1000
    L = _logits(T, E, seed=31 + zipf, zipf=zipf)
    b = (np.random.default_rng(32).standard_normal(E) * 0.3).astype(np.float32)
    print(f"full-size balance case zipf={zipf}", flush=True)
    idx, w, alpha = _check_qb_route(moe, dev, L, b, k)
    hist = _check_hist(moe, dev, L, gu.host(alpha).numpy(), k, lo, width, nb)
    new = moe.moe_qb_update(hist, k, lo, width, torch.from_numpy(b).to(dev))
    torch.cuda.synchronize()
    ref = bal.qb_update(gu.host(hist).to(torch.int64).numpy(), k, lo, width, b)
    assert np.array_equal(gu.host(new).numpy(), ref)
    _check_aux(moe, dev, L)
