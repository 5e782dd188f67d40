"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Sizes span several tiles with ragged tails (T not a multiple of the gate GEMM's
256-token tile, E not a multiple of 64, experts with more rows than one 192-row
m-tile, empty experts) plus the degenerate cases (T = 1, E = k = 1, k = E).
"""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as orc
from synthetic import CONFIGS, make_inputs, scaled_config
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


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------- top-k

def _planted_logits(T, E, seed):
    r = np.random.default_rng(seed)
    L = r.integers(-3, 4, size=(T, E)).astype(np.float32)  # many exact ties
    L[0] = 0.0
    if T > 1:
        L[1, ::2] = -0.0
    if T > 2:
        L[2] = r.standard_normal(E).astype(np.float32)
        if E >= 4:
            L[2, E // 2] = -np.inf
    if T > 3:
        L[3] = 1.0
        L[3, E - 1] = 1.0000001
    return L


@pytest.mark.parametrize("T,E,k", [(37, 8, 2), (70, 64, 8), (33, 100, 7), (9, 256, 4), (5, 896, 16),
                                   (4, 1024, 64), (3, 1, 1), (6, 65, 64)])
def test_topk_softmax_planted_ties(dev, moe, T, E, k):
    L = _planted_logits(T, E, seed=T * 1000 + E)
    idx, w = moe.moe_topk_softmax(torch.from_numpy(L).to(dev), k)
    _sync()
    gu.check_route(torch.from_numpy(L), idx, w, k)
    gi = idx.cpu().numpy()
    assert list(gi[0]) == list(range(k)), "all-zero row must pick experts 0..k-1"


def _zero_threshold_logits(E):
    """Rows whose k-th largest lane maximum (lane = id % 64) is exactly 0 or a negative
    denormal, with -0.0, +0.0 and denormals of both signs around it: the selection must
    tie -0 with +0 (lower id first) and keep a denormal apart from 0."""
    den = np.float32(1e-40)       # a float32 denormal
    tiny = np.float32(1.4e-45)    # the smallest one
    rows = []
    a = np.full(E, -1.0, np.float32)
    a[0:20] = 0.0                 # 20 lanes whose maximum is 0 ...
    a[1:20:2] = -0.0              # ... half of them -0
    a[64:84:3] = -0.0             # more zeros in the same lanes (higher ids)
    a[20:25] = den                # 5 lanes above 0
    a[30:40] = -den               # negative denormals: below every zero
    rows.append(a)
    b = np.full(E, -1.0, np.float32)
    b[0:10] = 0.0                 # 10 lanes at 0 or above ...
    b[3] = tiny
    b[5] = -0.0
    b[10:22] = -tiny              # ... then 12 lanes at the largest negative denormal
    b[64 + 10:64 + 14] = -tiny    # ties on it in those lanes, higher ids
    b[22:30] = -den
    rows.append(b)
    c = -np.abs(a)                # all non-positive: zeros of both signs are the largest
    rows.append(c)
    return np.stack(rows)


@pytest.mark.parametrize("E,k", [(896, 16), (128, 8), (100, 12)])
def test_topk_threshold_at_zero_and_denormals(dev, moe, E, k):
    L = _zero_threshold_logits(E)
    idx, w = moe.moe_topk_softmax(torch.from_numpy(L).to(dev), k)
    _sync()
    gu.check_route(torch.from_numpy(L), idx, w, k)


@pytest.mark.parametrize("E,k", [(896, 16), (130, 8)])
def test_topk_rows_mostly_minus_inf(dev, moe, E, k):
    """Fewer finite scores than k: the k-th lane maximum is -inf, and the -inf ties go to the lower ids."""
    r = np.random.default_rng(E + k)
    L = np.full((4, E), -np.inf, np.float32)
    for t, n_finite in enumerate([0, 1, k // 2, k - 1]):
        pos = r.choice(E, size=n_finite, replace=False)
        L[t, pos] = r.standard_normal(n_finite).astype(np.float32)
    idx, w = moe.moe_topk_softmax(torch.from_numpy(L).to(dev), k)
    _sync()
    gi = idx.cpu().numpy()
    with np.errstate(invalid="ignore"):  # the all -inf row has no defined softmax; only ids are compared
        idx_ref, _, _ = orc.route(L.astype(np.float64), k)
    assert np.array_equal(gi, idx_ref), (gi, idx_ref)


def test_topk_nan_rows_still_give_distinct_ids(dev, moe):
    E, k = 96, 8
    L = np.random.default_rng(0).standard_normal((6, E)).astype(np.float32)
    L[0, :] = np.nan
    L[1, ::3] = np.nan
    idx, w = moe.moe_topk_softmax(torch.from_numpy(L).to(dev), k)
    _sync()
    gi = idx.cpu().numpy()
    for t in range(6):
        assert len(set(gi[t])) == k and gi[t].min() >= 0 and gi[t].max() < E
    # rows without NaN follow the oracle exactly
    gu.check_route(torch.from_numpy(L[2:]), idx[2:], w[2:], k)


# ------------------------------------------------------------------- route

ROUTE_CASES = [
    ("tiny", dict()),
    ("prefill", dict(T=200, d=256, E=40, k=4, h=128)),
    ("many_expert", dict(T=130, d=384, E=130, k=16, h=128)),
    ("skewed", dict(T=67, d=128, E=96, k=16, h=128)),
    ("decode", dict(T=1, d=7168, E=384, k=8, h=128)),
    # enough 256-token x 128-expert tiles for two rounds of the CUs: the 512-token tiles, without
    # a K split (bias in the GEMM's epilogue), a partial last token block and expert block
    ("skewed", dict(T=8411, d=256, E=1000, k=16, h=128)),
]
ROUTE_IDS = ["tiny", "prefill", "many_expert", "skewed", "decode", "skewed_tall_tiles"]


@pytest.mark.parametrize("base,over", ROUTE_CASES, ids=ROUTE_IDS)
def test_route_vs_oracle(dev, moe, base, over):
    cfg = scaled_config(base, **over) if over else CONFIGS[base]
    inp = make_inputs(cfg, experts=False)
    g = inp.to(dev)
    logits, idx, w = moe.moe_route(g.x, g.w_router, g.router_bias, cfg.k)
    _sync()
    gu.check_logits(logits, orc.gate_logits(inp.x, inp.w_router, inp.router_bias))
    gu.check_route(logits, idx, w, cfg.k)


def test_route_duplicated_gate_rows_tie_to_lower_id(dev, moe):
    cfg = scaled_config("prefill", T=50, d=256, E=16, k=4, h=128)
    inp = make_inputs(cfg, experts=False)
    wr = inp.w_router.clone()
    wr[5] = wr[2]
    wr[11] = wr[2]
    wr[7] = wr[0]
    logits, idx, w = moe.moe_route(inp.x.to(dev), wr.to(dev), None, cfg.k)
    _sync()
    lg = logits.cpu()
    assert torch.equal(lg[:, 5], lg[:, 2]) and torch.equal(lg[:, 11], lg[:, 2]), "identical gate rows must tie exactly"
    gu.check_route(lg, idx, w, cfg.k)


def test_route_zero_gate(dev, moe):
    T, d, E, k = 70, 128, 24, 5
    x = torch.randn(T, d).to(torch.bfloat16).to(dev)
    logits, idx, w = moe.moe_route(x, torch.zeros(E, d, device=dev), None, k)
    _sync()
    assert torch.all(logits == 0)
    assert torch.equal(idx.cpu(), torch.arange(k, dtype=torch.int32).repeat(T, 1))
    assert torch.all(w == 1.0 / k)


# ----------------------------------------------------------------- permute

def _random_idx(T, E, k, seed, skew=False):
    r = np.random.default_rng(seed)
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if skew:  # every token picks expert 0 (somewhere in its slots)
        for t in range(T):
            if 0 not in idx[t]:
                idx[t, r.integers(k)] = 0
    return idx


@pytest.mark.parametrize("T,E,k,skew", [(64, 8, 2, False), (300, 37, 4, False), (1, 5, 3, False),
                                        (1000, 64, 8, True), (2049, 256, 4, False), (777, 896, 16, False),
                                        (513, 1024, 2, True), (4000, 1024, 8, True)])
def test_permute_vs_oracle(dev, moe, T, E, k, skew):
    d = 256
    idx = _random_idx(T, E, k, seed=T + E, skew=skew)
    x = torch.randn(T, d).to(torch.bfloat16)
    off, row_of, row_src, x_perm = moe.moe_permute(x.to(dev), torch.from_numpy(idx).to(dev), E)
    _sync()
    _, _, rs = gu.check_permutation(off, row_of, row_src, idx, E)
    assert torch.equal(x_perm.cpu(), x[torch.from_numpy(rs)]), "x_perm is not x[row_src]"


@pytest.mark.parametrize("d", [640, 1152])
def test_permute_gather_rows_spanning_blocks(dev, moe, d):
    """x_perm rows wider than one 512-element gather block, with a partial last block."""
    T, E, k = 77, 9, 3
    idx = _random_idx(T, E, k, seed=d)
    x = torch.randn(T, d).to(torch.bfloat16)
    off, row_of, row_src, x_perm = moe.moe_permute(x.to(dev), torch.from_numpy(idx).to(dev), E)
    _sync()
    _, _, rs = gu.check_permutation(off, row_of, row_src, idx, E)
    assert torch.equal(x_perm.cpu(), x[torch.from_numpy(rs)]), "x_perm is not x[row_src]"


def test_permute_skips_out_of_range_ids(dev, moe):
    T, E, k, d = 40, 6, 2, 128
    idx = _random_idx(T, E, k, seed=3)
    idx[3, 1] = -1
    idx[17, 0] = E
    x = torch.randn(T, d).to(torch.bfloat16)
    off, row_of, row_src, x_perm = moe.moe_permute(x.to(dev), torch.from_numpy(idx).to(dev), E)
    _sync()
    ro = row_of.cpu().numpy()
    assert ro[3, 1] == -1 and ro[17, 0] == -1
    assert off.cpu().numpy()[E] == T * k - 2
    valid = (idx >= 0) & (idx < E)
    rs = row_src.cpu().numpy()
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                assert rs[ro[t, j]] == t


# -------------------------------------------------------------- expert FFN

FFN_CASES = [
    # (T, d, E, k, h, skew): skew sends every token to expert 0 -> T rows, several 192-row m-tiles
    (64, 128, 8, 2, 256, False),
    (300, 256, 12, 4, 384, False),
    (37, 384, 5, 2, 128, True),
    (260, 128, 3, 1, 128, True),
    (600, 256, 3, 1, 256, True),   # 600 rows on expert 0: four m-tiles of 150 rows
    (1, 256, 4, 2, 256, False),
    (129, 512, 64, 8, 256, False),
]


@pytest.mark.parametrize("gathered", [False, True], ids=["x_perm", "x_row_src"])
@pytest.mark.parametrize("T,d,E,k,h,skew", FFN_CASES)
def test_expert_ffn_vs_oracle(dev, moe, T, d, E, k, h, skew, gathered):
    cfg = scaled_config("tiny", T=T, d=d, E=E, k=k, h=h, seed=T + d)
    inp = make_inputs(cfg)
    idx = _random_idx(T, E, k, seed=T, skew=skew)
    off, row_of, row_src = orc.permute(idx, E)
    x_perm = inp.x[torch.from_numpy(row_src)]
    off_d = torch.from_numpy(off.astype(np.int32)).to(dev)
    w = gu.packed(inp.w_gate.to(dev), inp.w_up.to(dev), inp.w_down.to(dev))
    if gathered:  # rows read from x through row_src inside the GEMM
        h_act, y_rows = moe.moe_expert_ffn(inp.x.to(dev), off_d, *w, T, k,
                                           a_rows=torch.from_numpy(row_src.astype(np.int32)).to(dev))
        h_ref, y_ref = moe.moe_expert_ffn(x_perm.to(dev), off_d, *w, T, k)
        _sync()
        assert torch.equal(h_act, h_ref) and torch.equal(y_rows, y_ref), "gathered rows differ from x_perm rows"
    else:
        h_act, y_rows = moe.moe_expert_ffn(x_perm.to(dev), off_d, *w, T, k)
    _sync()
    H_ref, Y_ref = orc.expert_ffn(x_perm, off, inp.w_gate, inp.w_up, inp.w_down)
    hg, yg = h_act.cpu(), y_rows.cpu()
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        gu.check_h_rows(hg[lo:hi], H_ref[lo:hi], what=f"H expert {e}")
        gu.check_y_rows(yg[lo:hi], Y_ref[lo:hi], H_ref[lo:hi], inp.w_down[e], what=f"Y expert {e}")


# ----------------------------------------------------------------- combine

@pytest.mark.parametrize("T,d,k", [(64, 128, 2), (333, 384, 4), (5, 7168, 16), (17, 256, 64), (1, 128, 1)])
def test_combine_vs_oracle(dev, moe, T, d, k):
    r = np.random.default_rng(T * k)
    E = max(k, 70)
    idx = _random_idx(T, E, k, seed=T + k)
    _, row_of, _ = orc.permute(idx, E)
    Y = torch.randn(T * k, d)
    w = torch.from_numpy(r.dirichlet(np.ones(k), size=T).astype(np.float32))
    out = moe.moe_combine(Y.to(dev), torch.from_numpy(row_of.astype(np.int32)).to(dev), w.to(dev))
    _sync()
    ref = orc.combine(Y, row_of, w)
    scale = np.abs(orc.f64(w))[:, :, None] * np.abs(orc.f64(Y))[row_of]
    bound = (k + 1) * 2.0 ** -23 * scale.sum(1) + 1e-30  # float32 sum of k exact products
    assert np.all(np.abs(orc.f64(out) - ref) <= bound)


# --------------------------------------------------------------- whole layer

def _forward_and_oracle(moe, dev, inp, cfg, **wover):
    g = inp.to(dev)
    ws = dict(w_gate=g.w_gate, w_up=g.w_up, w_down=g.w_down)
    ws.update({k_: v.to(dev) for k_, v in wover.items()})
    fwd = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    out = fwd(g.x, g.w_router, g.router_bias, *gu.packed(ws["w_gate"], ws["w_up"], ws["w_down"]))
    _sync()
    host_w = dict(w_gate=inp.w_gate, w_up=inp.w_up, w_down=inp.w_down)
    host_w.update(wover)
    logits = fwd.intermediate("logits").cpu()
    ref = orc.forward(inp.x, inp.w_router, inp.router_bias, host_w["w_gate"], host_w["w_up"], host_w["w_down"],
                      cfg.k, logits=logits)
    return fwd, out, ref


LAYER_CASES = [
    ("tiny", dict()),
    ("prefill", dict(T=333, d=256, E=20, k=4, h=256)),
    ("decode", dict(T=5, d=1024, E=48, k=8, h=512)),
    ("many_expert", dict(T=190, d=256, E=130, k=16, h=128)),
    ("skewed", dict(T=300, d=256, E=96, k=16, h=128)),
]


def _random_layer_shape(seed):
    """A seeded layer shape: ragged token counts, widths of 1 to 5 K blocks, any expert count up to 160,
    every top-k up to 16, with and without the skewed workload's gate bias."""
    r = np.random.default_rng(1000 + seed)
    E = int(r.integers(1, 161))
    k = int(r.integers(1, min(E, 16) + 1))
    return ("skewed" if seed % 2 else "prefill"), dict(T=int(r.integers(1, 601)), d=int(r.choice([128, 256, 384, 640])),
                                                       E=E, k=k, h=int(r.choice([128, 256, 384])))


@pytest.mark.parametrize("seed", range(24))
def test_forward_random_shapes(dev, moe, seed):
    base, over = _random_layer_shape(seed)
    cfg = scaled_config(base, seed=50 + seed, **over)
    print(f"[random layer] seed {seed}: {base} {over}", flush=True)
    inp = make_inputs(cfg)
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    gu.check_logits(ref["logits"], orc.gate_logits(inp.x, inp.w_router, inp.router_bias))
    gu.check_route(fwd.intermediate("logits"), fwd.intermediate("topk_idx"), fwd.intermediate("topk_w"), cfg.k)
    gu.check_permutation(fwd.intermediate("expert_offsets"), fwd.intermediate("row_of"),
                         fwd.intermediate("row_src"), ref["idx"], cfg.E)
    gu.check_layer(out, ref["out"])


@pytest.mark.parametrize("base,over", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_forward_vs_oracle(dev, moe, base, over):
    cfg = scaled_config(base, **over) if over else CONFIGS[base]
    inp = make_inputs(cfg)
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    gu.check_logits(ref["logits"], orc.gate_logits(inp.x, inp.w_router, inp.router_bias))
    gu.check_route(fwd.intermediate("logits"), fwd.intermediate("topk_idx"), fwd.intermediate("topk_w"), cfg.k)
    gu.check_permutation(fwd.intermediate("expert_offsets"), fwd.intermediate("row_of"),
                         fwd.intermediate("row_src"), ref["idx"], cfg.E)
    gu.check_layer(out, ref["out"])
    # the forward pass (gather fused into the gate/up pass) equals the four calls
    # made one by one with an explicit x_perm, bit for bit
    g = inp.to(dev)
    logits, idx, w = moe.moe_route(g.x, g.w_router, g.router_bias, cfg.k)
    off, row_of, row_src, x_perm = moe.moe_permute(g.x, idx, cfg.E)
    _sync()
    assert torch.equal(x_perm.cpu(), inp.x[torch.from_numpy(ref["row_src"])])
    h_act, y_rows = moe.moe_expert_ffn(x_perm, off, *gu.packed(g.w_gate, g.w_up, g.w_down), cfg.T, cfg.k)
    out2 = moe.moe_combine(y_rows, row_of, w)
    _sync()
    assert torch.equal(out2, out)
    assert torch.equal(h_act, fwd.intermediate("h_act"))


def test_forward_identical_experts_is_dense_ffn(dev, moe):
    cfg = scaled_config("prefill", T=150, d=256, E=12, k=4, h=256)
    inp = make_inputs(cfg)
    for t in (inp.w_gate, inp.w_up, inp.w_down):
        t[:] = t[0]
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    X = torch.as_tensor(orc.f64(inp.x))
    dense = torch.nn.functional.silu(X @ torch.as_tensor(orc.f64(inp.w_gate[0])).t()) * \
        (X @ torch.as_tensor(orc.f64(inp.w_up[0])).t())
    dense = (dense @ torch.as_tensor(orc.f64(inp.w_down[0])).t()).numpy()
    gu.check_layer(out, dense, what="identical experts vs dense FFN")


def test_forward_k_equals_E_is_dense_mixture(dev, moe):
    cfg = scaled_config("tiny", T=70, d=128, E=6, k=6, h=128)
    inp = make_inputs(cfg)
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    p = orc.softmax(fwd.intermediate("logits").cpu())
    mix = np.zeros((cfg.T, cfg.d))
    for e in range(cfg.E):
        _, Ye = orc.expert_swiglu(inp.x, inp.w_gate[e], inp.w_up[e], inp.w_down[e])
        mix += p[:, e:e + 1] * Ye
    gu.check_layer(out, mix, what="k = E vs dense softmax mixture")


def test_forward_single_expert(dev, moe):
    cfg = scaled_config("tiny", T=45, d=256, E=1, k=1, h=384)
    inp = make_inputs(cfg)
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    assert torch.all(fwd.intermediate("topk_w") == 1.0)
    gu.check_layer(out, ref["out"])


def test_forward_zero_down_gives_zero(dev, moe):
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg)
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg, w_down=torch.zeros_like(inp.w_down))
    assert torch.all(out == 0)


def test_forward_one_token_and_all_tokens_on_one_expert(dev, moe):
    # T = 1
    cfg = scaled_config("decode", T=1, d=512, E=40, k=8, h=256)
    inp = make_inputs(cfg)
    _, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    gu.check_layer(out, ref["out"])
    # a bias that sends every token to expert 3 first: that expert gets T rows (several m-tiles)
    cfg = scaled_config("prefill", T=400, d=256, E=16, k=2, h=128)
    inp = make_inputs(cfg)
    inp.router_bias = torch.zeros(cfg.E)
    inp.router_bias[3] = 50.0
    fwd, out, ref = _forward_and_oracle(moe, dev, inp, cfg)
    offs = fwd.intermediate("expert_offsets").cpu().numpy()
    assert offs[4] - offs[3] == cfg.T
    gu.check_layer(out, ref["out"])


def test_forward_deterministic_and_token_equivariant(dev, moe):
    cfg = scaled_config("prefill", T=257, d=256, E=24, k=4, h=256)
    inp = make_inputs(cfg)
    g = inp.to(dev)
    fwd = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    w = gu.packed(g.w_gate, g.w_up, g.w_down)
    a = fwd(g.x, g.w_router, None, *w).clone()
    b = fwd(g.x, g.w_router, None, *w).clone()
    _sync()
    assert torch.equal(a, b), "two runs differ"
    perm = torch.from_numpy(np.random.default_rng(0).permutation(cfg.T)).to(dev)
    c = fwd(g.x[perm].contiguous(), g.w_router, None, *w)
    _sync()
    assert torch.equal(c, a[perm]), "permuting tokens does not permute the output rows"


def test_forward_zero_tokens(dev, moe):
    fwd = moe.MoEForward(0, 128, 8, 2, 256, dev)
    inp = make_inputs(CONFIGS["tiny"]).to(dev)
    out = fwd(torch.empty(0, 128, dtype=torch.bfloat16, device=dev), inp.w_router, None,
              *gu.packed(inp.w_gate, inp.w_up, inp.w_down))
    _sync()
    assert out.shape == (0, 128)
