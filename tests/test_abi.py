"""CPU tests of the C ABI: the library loads, exports every declared call, and
rejects bad arguments on the host before anything is launched (no GPU needed:
each call here fails validation before its first HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "libmoe.so")


def _ensure_built():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._build_module().build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    from sparse_mixture_experts_fp32_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_workspace_bytes", "moe_status_str", "moe_last_error", "moe_aux_loss",
              "moe_qb_route", "moe_qb_histogram", "moe_qb_update", "moe_latent_forward",
              "moe_latent_workspace_bytes", "moe_latent_ws_offset", "moe_combine_rmsnorm",
              "moe_mx_quantize_weights", "moe_mx_quantize_rows", "moe_mx_expert_ffn", "moe_mx_forward",
              "moe_mx_forward_ws_offset", "moe_mx_expert_gate_up", "moe_mx_expert_down",
              "moe_pack_weights", "moe_permute_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", nm))
    assert set(declared_functions()) <= exported


def test_probe_library_exports_its_header():
    """libmoe_probe.so (the ceiling probes) exports every call include/moe_probe.h declares and
    rejects bad arguments before launching anything."""
    _ensure_built()
    path = os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "libmoe_probe.so")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"^\s*int\s+(moe_probe_[a-z_]+)\s*\(", text, flags=re.M)))
    assert names == ["moe_probe_copy", "moe_probe_dma_read", "moe_probe_mfma", "moe_probe_read", "moe_probe_read_tiles"]
    L = ctypes.CDLL(path)
    for n in names:
        assert hasattr(L, n), n
    a = ctypes.c_void_p(4096)
    sz = ctypes.c_size_t
    assert L.moe_probe_read(None, sz(16), a, None) == -1
    assert L.moe_probe_read(a, sz(15), a, None) == -1
    assert L.moe_probe_read_tiles(a, sz(24), a, None) == -1       # not a multiple of 16
    assert L.moe_probe_read_tiles(a, sz(16), None, None) == -1
    assert L.moe_probe_dma_read(a, sz(16), a, None) == -1          # not a whole 32 KiB stage
    assert L.moe_probe_copy(a, ctypes.c_void_p(4096 + 16), sz(64), None) == -1  # overlapping
    assert L.moe_probe_mfma(6, 10, a, None) == -1                  # waves not a multiple of 4
    assert L.moe_probe_mfma(8, 40000, a, None) == -1               # beyond the exact range


def test_status_strings(lib):
    L = lib.lib
    assert L.moe_abi_version() == lib.ABI_VERSION == 10
    assert L.moe_status_str(0) == b"ok"
    for s in range(1, 5):
        assert L.moe_status_str(s) and L.moe_status_str(s) != b"ok"
    assert L.moe_status_str(99) == b"unknown status"


GOOD = dict(T=64, d=128, E=8, k=2, h=256)


def _shape(lib, **kw):
    p = dict(GOOD)
    p.update(kw)
    return lib.shape(p["T"], p["d"], p["E"], p["k"], p["h"])


@pytest.mark.parametrize("bad,status", [
    (dict(T=-1), 1), (dict(E=0), 1), (dict(E=1025), 1), (dict(k=0), 1), (dict(k=9), 1),
    (dict(E=100, k=65), 1), (dict(d=96), 1), (dict(d=0), 1), (dict(h=200), 1), (dict(h=-128), 1),
    (dict(T=2**28, k=8), 2),
])
def test_bad_shapes_rejected(lib, bad, status):
    s = _shape(lib, **bad)
    fake = ctypes.c_void_p(4096)
    st = lib.lib.moe_route(ctypes.byref(s), fake, fake, None, fake, fake, fake, fake, 1 << 30, None)
    assert st == status, lib.lib.moe_last_error()
    assert lib.lib.moe_last_error()
    assert lib.lib.moe_workspace_bytes(ctypes.byref(s), 2) == 0


def test_null_and_misaligned_pointers_rejected(lib):
    s = _shape(lib)
    a = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 2)
    L = lib.lib
    assert L.moe_route(ctypes.byref(s), None, a, None, a, a, a, a, 1 << 30, None) == 1
    assert b"x is NULL" in L.moe_last_error()
    assert L.moe_route(ctypes.byref(s), mis, a, None, a, a, a, a, 1 << 30, None) == 1
    assert b"aligned" in L.moe_last_error()
    assert L.moe_route(ctypes.byref(s), a, a, mis, a, a, a, a, 1 << 30, None) == 1
    assert L.moe_topk_softmax(ctypes.byref(s), None, a, a, None) == 1
    assert L.moe_combine(ctypes.byref(s), a, a, None, a, None) == 1
    assert L.moe_expert_ffn(ctypes.byref(s), a, None, a, a, a, None, a, a, a, 1 << 20, None) == 1
    assert L.moe_expert_ffn(ctypes.byref(s), None, a, a, a, a, a, a, a, a, 1 << 20, None) == 1
    assert L.moe_expert_ffn(ctypes.byref(s), a, mis, a, a, a, a, a, a, a, 1 << 20, None) == 1
    assert L.moe_expert_gate_up(ctypes.byref(s), a, None, a, a, None, a, a, 1 << 20, None) == 1
    # moe_permute: x_perm may be NULL (no gather; x is then not needed), but not misaligned
    assert L.moe_permute(ctypes.byref(s), a, a, a, a, a, mis, a, 1 << 20, None) == 1
    assert L.moe_permute(ctypes.byref(s), None, a, a, a, a, a, a, 1 << 20, None) == 1
    assert L.moe_forward(ctypes.byref(s), a, a, None, a, a, a, None, a, 1 << 30, None) == 1
    assert L.moe_route(None, a, a, None, a, a, a, a, 1 << 30, None) == 1


def test_noalloc_permute_checks_arguments(lib):
    """moe_permute_noalloc validates like moe_permute (minus the workspace) before it looks
    up its scratch array or launches anything."""
    s = _shape(lib)
    a = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 2)
    L = lib.lib
    assert L.moe_permute_noalloc(ctypes.byref(s), a, a, a, a, a, mis, None) == 1
    assert b"x_perm" in L.moe_last_error()
    assert L.moe_permute_noalloc(ctypes.byref(s), None, a, a, a, a, a, None) == 1
    assert L.moe_permute_noalloc(ctypes.byref(s), a, None, a, a, a, None, None) == 1
    assert L.moe_permute_noalloc(ctypes.byref(s), a, a, None, a, a, None, None) == 1
    assert L.moe_permute_noalloc(ctypes.byref(s), a, a, a, a, None, None, None) == 1
    assert L.moe_permute_noalloc(None, a, a, a, a, a, None, None) == 1
    assert L.moe_permute_noalloc(ctypes.byref(_shape(lib, E=1025)), a, a, a, a, a, None, None) == 1
    # the largest count matrix of any valid shape fits the fixed scratch
    big = _shape(lib, T=4_000_000, E=1024, k=16)
    assert L.moe_workspace_bytes(ctypes.byref(big), 0) == 1024 * 32 * 4 == 131072


def test_workspace_checks(lib):
    s = _shape(lib)
    L = lib.lib
    a = ctypes.c_void_p(4096)
    need_p = lib.workspace_bytes(s, lib.MOE_CALL_PERMUTE)
    need_f = lib.workspace_bytes(s, lib.MOE_CALL_EXPERT_FFN)
    need_fw = lib.workspace_bytes(s, lib.MOE_CALL_FORWARD)
    need_r = lib.workspace_bytes(s, lib.MOE_CALL_ROUTE)
    assert need_r >= 3 * 2 * GOOD["E"] * GOOD["d"] and need_r % 256 == 0
    assert L.moe_route(ctypes.byref(s), a, a, None, a, a, a, None, need_r, None) == 3
    assert L.moe_route(ctypes.byref(s), a, a, None, a, a, a, a, need_r - 1, None) == 3
    assert need_p > 0 and need_f > 0 and need_fw > 0
    assert need_p % 256 == 0 and need_f % 256 == 0 and need_fw % 256 == 0
    assert L.moe_permute(ctypes.byref(s), a, a, a, a, a, a, None, need_p, None) == 3
    assert L.moe_permute(ctypes.byref(s), a, a, a, a, a, a, a, need_p - 1, None) == 3
    assert L.moe_permute(ctypes.byref(s), a, a, a, a, a, a, ctypes.c_void_p(4096 + 16), need_p, None) == 3
    assert L.moe_expert_ffn(ctypes.byref(s), a, None, a, a, a, a, a, a, a, need_f - 1, None) == 3
    assert L.moe_forward(ctypes.byref(s), a, a, None, a, a, a, a, a, need_fw - 256, None) == 3
    assert L.moe_workspace_bytes(ctypes.byref(s), 7) == 0


def test_route_workspace_follows_the_k_split(lib):
    """The router's workspace is its three bf16 weight parts plus, when K is split, one float32
    partial sum per K range: 4 ranges at prefill (64 token x expert tiles), 32 at decode (3 tiles),
    none once the tiles fill the CUs (many_expert: 512-token tiles, one round)."""
    for (T, d, E), S in [((8192, 7168, 256), 4), ((128, 7168, 384), 32), ((16384, 7168, 896), 1),
                         ((6144, 1024, 1024), 1)]:
        s = lib.shape(T, d, E, 4, 128)
        parts = 3 * 2 * ((E + 15) // 16 * 16) * d
        want = (parts + 255) // 256 * 256 + (4 * S * T * E if S > 1 else 0)
        assert lib.workspace_bytes(s, lib.MOE_CALL_ROUTE) == (want + 255) // 256 * 256, (T, d, E)


def test_forward_workspace_layout(lib):
    """Every intermediate fits inside the forward workspace, aligned, without overlap."""
    for cfg in [GOOD, dict(T=8192, d=7168, E=256, k=4, h=2048), dict(T=16384, d=7168, E=896, k=16, h=1024),
                dict(T=1, d=128, E=1, k=1, h=128)]:
        s = lib.shape(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["h"])
        total = lib.workspace_bytes(s, lib.MOE_CALL_FORWARD)
        T, d, E, k, h = (cfg[c] for c in "TdEkh")
        sizes = [4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k, 2 * T * k * h, 4 * T * k * d]
        ns = len(lib.FWD_SLOTS)
        assert ns == len(sizes)
        offs = [lib.forward_ws_offset(s, i) for i in range(ns)]
        for i in range(ns):
            assert offs[i] % 256 == 0
            assert offs[i] + sizes[i] <= total
            if i + 1 < ns:
                assert offs[i] + sizes[i] <= offs[i + 1]
    with pytest.raises(lib.MoEError):
        lib.forward_ws_offset(lib.shape(64, 128, 8, 2, 256), len(lib.FWD_SLOTS))


def test_zero_tokens_is_a_noop(lib):
    s = _shape(lib, T=0)
    L = lib.lib
    assert L.moe_route(ctypes.byref(s), None, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_combine(ctypes.byref(s), None, None, None, None, None) == 0
    assert L.moe_forward(ctypes.byref(s), None, None, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_expert_ffn(ctypes.byref(s), None, None, None, None, None, None, None, None, None, 0, None) == 0


def test_balance_calls_reject_bad_arguments(lib):
    L = lib.lib
    a = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 4)
    s = _shape(lib)
    f = ctypes.c_float
    # Quantile Balancing needs k < E and k <= 63
    for bad in (dict(k=8, E=8), dict(E=100, k=64)):
        sb = _shape(lib, **bad)
        assert L.moe_qb_route(ctypes.byref(sb), a, a, a, a, a, None) == 1
        assert b"k < E" in L.moe_last_error()
        assert L.moe_qb_histogram(ctypes.byref(sb), a, a, f(-8.0), f(0.01), 1000, a, None) == 1
        assert L.moe_qb_update(ctypes.byref(sb), a, f(-8.0), f(0.01), 1000, a, a, None) == 1
    assert L.moe_qb_route(ctypes.byref(s), a, None, a, a, a, None) == 1
    assert L.moe_qb_route(ctypes.byref(s), a, a, a, a, mis, None) == 1
    for lo, width, nb in [(float("nan"), 0.01, 10), (0.0, 0.0, 10), (0.0, -1.0, 10), (0.0, float("inf"), 10),
                          (float("-inf"), 1.0, 10), (0.0, 0.01, 0), (0.0, 0.01, 4097)]:
        assert L.moe_qb_histogram(ctypes.byref(s), a, a, f(lo), f(width), nb, a, None) == 1
        assert L.moe_qb_update(ctypes.byref(s), a, f(lo), f(width), nb, a, a, None) == 1
    assert L.moe_qb_histogram(ctypes.byref(s), a, a, f(0.0), f(0.01), 100, None, None) == 1
    assert L.moe_qb_update(ctypes.byref(s), a, f(0.0), f(0.01), 100, None, a, None) == 1
    assert L.moe_aux_loss(ctypes.byref(s), None, a, a, a, 1 << 20, None) == 1
    need = lib.workspace_bytes(s, lib.MOE_CALL_AUX_LOSS)
    assert need >= 4 * GOOD["E"] + 8 * GOOD["E"] and need % 256 == 0
    assert L.moe_aux_loss(ctypes.byref(s), a, a, a, a, need - 1, None) == 3
    assert L.moe_aux_loss(ctypes.byref(s), a, a, a, None, need, None) == 3
    s0 = _shape(lib, T=0)
    assert L.moe_aux_loss(ctypes.byref(s0), None, None, None, None, 0, None) == 0
    assert L.moe_qb_route(ctypes.byref(s0), None, None, None, None, None, None) == 0


def test_latent_shape_checks_and_layout(lib):
    L = lib.lib
    a = ctypes.c_void_p(4096)
    f = ctypes.c_float
    good = dict(T=64, d=256, l=128, E=8, k=2, h=256, n_shared=2, h_shared=128)

    def ls(**kw):
        p = dict(good)
        p.update(kw)
        return lib.latent_shape(*(p[c] for c in ("T", "d", "l", "E", "k", "h", "n_shared", "h_shared")))

    for bad, status in [(dict(l=96), 1), (dict(d=100), 1), (dict(n_shared=9), 1), (dict(n_shared=-1), 1),
                        (dict(h_shared=0), 1), (dict(l=8192 + 128), 2), (dict(k=9), 1), (dict(T=-1), 1)]:
        s = ls(**bad)
        assert L.moe_latent_workspace_bytes(ctypes.byref(s)) == 0
        assert L.moe_latent_forward(ctypes.byref(s), a, a, None, a, a, a, a, a, f(1e-6), a, a, a, a, a, a,
                                    1 << 40, None) == status, (bad, L.moe_last_error())
    s = ls()
    need = lib.latent_workspace_bytes(s)
    args = [a, a, None, a, a, a, a, a, f(1e-6), a, a, a, a, a]
    assert L.moe_latent_forward(ctypes.byref(s), *args, a, need - 1, None) == 3
    assert L.moe_latent_forward(ctypes.byref(s), *args[:8], f(-1.0), *args[9:], a, need, None) == 1
    assert L.moe_latent_forward(ctypes.byref(s), *args[:10], None, *args[11:], a, need, None) == 1
    s0 = ls(n_shared=0, h_shared=0)
    args0 = [a, a, None, a, a, a, a, a, f(1e-6), a, None, None, None, a]
    assert L.moe_latent_forward(ctypes.byref(s0), *args0, a, 1, None) == 3  # shared may be NULL; ws too small
    # every slot inside the workspace, aligned, in order, sized as documented
    for cfg in [good, dict(good, n_shared=0, h_shared=0),
                dict(T=16384, d=7168, l=3584, E=896, k=16, h=1024, n_shared=2, h_shared=2048)]:
        s = ls(**cfg)
        total = lib.latent_workspace_bytes(s)
        T, d, l, E, k, h, S, hs = (cfg[c] for c in ("T", "d", "l", "E", "k", "h", "n_shared", "h_shared"))
        sizes = [4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k, 2 * T * l, 2 * T * k * h,
                 4 * T * k * l, 2 * T * l, 2 * S * T * hs, 4 * S * T * d]
        assert len(sizes) == len(lib.LAT_SLOTS)
        offs = [lib.latent_ws_offset(s, i) for i in range(len(sizes))]
        for i in range(len(sizes)):
            assert offs[i] % 256 == 0 and offs[i] + sizes[i] <= total
            if i + 1 < len(sizes):
                assert offs[i] + sizes[i] <= offs[i + 1]
    # combine_rmsnorm: width limit and eps
    s = _shape(lib, d=8192 + 128)
    assert L.moe_combine_rmsnorm(ctypes.byref(s), a, a, a, a, f(1e-6), None, a, None) == 2
    s = _shape(lib)
    assert L.moe_combine_rmsnorm(ctypes.byref(s), a, a, a, a, f(float("nan")), None, a, None) == 1
    assert L.moe_combine_rmsnorm(ctypes.byref(s), a, a, a, None, f(1e-6), None, a, None) == 1
    assert L.moe_combine_rmsnorm(ctypes.byref(s), a, a, a, a, f(1e-6), ctypes.c_void_p(4100), a, None) == 1


def test_mx_calls_check_arguments(lib):
    L = lib.lib
    a = ctypes.c_void_p(4096)
    # d and h must be multiples of 512 for the MX path
    s = _shape(lib, d=256, h=512)
    assert L.moe_mx_forward(ctypes.byref(s), a, a, None, a, a, a, a, a, a, a, a, 1 << 30, None) == 2
    assert L.moe_workspace_bytes(ctypes.byref(s), lib.MOE_CALL_MX_FORWARD) == 0
    # the MX grouped GEMM addresses its MXFP8 rows with 32-bit offsets: T * k * max(d, h) < 2^32
    s = _shape(lib, T=1 << 20, d=4096, h=512, E=8, k=1)
    assert L.moe_mx_expert_gate_up(ctypes.byref(s), a, a, None, a, a, a, a, a, a, a, 1 << 20, None) == 2
    assert L.moe_mx_expert_down(ctypes.byref(s), a, a, a, a, a, a, a, 1 << 20, None) == 2
    s = _shape(lib, d=512, h=512)
    need = lib.workspace_bytes(s, lib.MOE_CALL_MX_FORWARD)
    assert need > 0 and need % 256 == 0
    assert L.moe_mx_forward(ctypes.byref(s), a, a, None, a, a, a, a, a, a, a, a, need - 1, None) == 3
    assert L.moe_mx_forward(ctypes.byref(s), a, a, None, a, None, a, a, a, a, a, a, need, None) == 1
    assert L.moe_mx_expert_ffn(ctypes.byref(s), a, a, None, a, a, a, a, a, a, a, a, None, a, a, a, 1 << 20,
                               None) == 1
    assert L.moe_mx_expert_gate_up(ctypes.byref(s), a, a, None, a, a, a, a, a, None, a, 1 << 20, None) == 1
    assert L.moe_mx_expert_down(ctypes.byref(s), a, a, a, a, a, a, a, 10, None) == 3
    assert L.moe_mx_quantize_weights(2, 16, 256, a, a, a, None) == 1       # K not a multiple of 512
    assert L.moe_mx_quantize_weights(2, 16, 512, None, a, a, None) == 1
    assert L.moe_mx_quantize_weights(0, 16, 512, None, None, None, None) == 0
    assert L.moe_mx_quantize_rows(4, 48, a, 0, a, a, None) == 1             # K not a multiple of 32
    assert L.moe_mx_quantize_rows(0, 64, None, 0, None, None, None) == 0
    T, d, E, k, h = 64, 512, 8, 2, 512
    sizes = [4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k, T * d, T * d // 32,
             4 * T * k * h, T * k * h, T * k * h // 32, 4 * T * k * d]
    s = lib.shape(T, d, E, k, h)
    total = lib.workspace_bytes(s, lib.MOE_CALL_MX_FORWARD)
    assert len(sizes) == len(lib.MX_SLOTS)
    offs = [lib.mx_forward_ws_offset(s, i) for i in range(len(sizes))]
    for i in range(len(sizes)):
        assert offs[i] % 256 == 0 and offs[i] + sizes[i] <= total
        if i + 1 < len(sizes):
            assert offs[i] + sizes[i] <= offs[i + 1]


def test_pack_weights_checks_arguments(lib):
    L = lib.lib
    a, b = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    assert L.moe_pack_weights(2, 24, 128, a, b, None) == 1     # N not a multiple of 16
    assert L.moe_pack_weights(2, 32, 80, a, b, None) == 1      # K not a multiple of 32
    assert L.moe_pack_weights(2, 32, 128, a, a, None) == 1     # in place
    assert L.moe_pack_weights(2, 32, 128, a, ctypes.c_void_p(4096 + 2 * 32 * 128 * 2 - 16), None) == 1  # overlap
    assert L.moe_pack_weights(2, 32, 128, None, b, None) == 1
    assert L.moe_pack_weights(0, 32, 128, None, None, None) == 0


def test_one_weight_format(lib):
    """The layer calls take packed weights; no second, row-major entry point exists."""
    names = declared_functions()
    assert not [n for n in names if n.endswith("_packed")], names
    raw = ctypes.CDLL(LIB)
    for n in ("moe_forward_packed", "moe_expert_gate_up_packed", "moe_expert_down_packed",
              "moe_latent_forward_packed"):
        assert not hasattr(raw, n), n
