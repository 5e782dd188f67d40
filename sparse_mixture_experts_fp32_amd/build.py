"""Build libmoe.so and libmoe_probe.so (gfx950) in-tree with hipcc.

    python -m sparse_mixture_experts_fp32_amd.build [--sanitize]

Compiles the layer's sources under csrc/ for gfx950 only and links
libmoe.so next to this file; the ceiling probes (csrc/probe.hip) go into
libmoe_probe.so. Packed-fp32 instruction selection is switched off for all
device code.

--sanitize builds libmoe_san.so instead: the same sources with the host code
(argument checks, workspace layout, launch set-up) under AddressSanitizer and
UndefinedBehaviorSanitizer; device code is built as usual. It is for running
the CPU-side ABI tests under the sanitizers (MOE_LIBRARY selects it, with the
sanitizer runtime preloaded).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
LIB_PROBE = os.path.join(PKG, "libmoe_probe.so")
LIB_SAN = os.path.join(PKG, "libmoe_san.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "permute.hip", "tiles.hip", "ffn_ring.hip", "combine.hip", "balance.hip", "latent.hip", "mx.hip", "moe_api.cpp"]
PROBE_SOURCES = ["probe.hip"]
# host-side sanitizers only (each -fsanitize= right after -Xarch_host: device code is built as usual)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
            "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _compile(hipcc: str, src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [hipcc, *COMMON, *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(hipcc: str, objs, lib: str, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = True, extra=()) -> str:
    """Compile all sources and link libmoe.so and libmoe_probe.so; returns libmoe.so's path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(hipcc, s, list(extra)), srcs)))
    _link(hipcc, [objs[s] for s in SOURCES], LIB)
    _link(hipcc, [objs[s] for s in PROBE_SOURCES], LIB_PROBE)
    if verbose:
        print(f"built {LIB} and {LIB_PROBE}")
    return LIB


def build_sanitized(verbose: bool = True) -> str:
    """libmoe_san.so: the layer's sources with host-side ASan + UBSan; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, SANITIZE, ".san"), SOURCES))
    _link(hipcc, objs, LIB_SAN, ["-fsanitize=address,undefined"])
    if verbose:
        print(f"built {LIB_SAN}")
    return LIB_SAN


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into a host process)."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return res.stdout.strip()


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
