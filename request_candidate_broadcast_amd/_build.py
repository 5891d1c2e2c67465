"""Builds libikbo.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libikbo.so")
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libikbo_probe.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("IKBO_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # keep the compiler from forming packed-fp32 VALU ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel whose host launch stub was not emitted fails here, not at dlopen
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, out)


def build_probe(verbose: bool = True) -> str:
    """Compile probe/*.hip (the roofline ceiling probes) into libikbo_probe.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip"))
    _link([_compile(s) for s in srcs], PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = True) -> str:
    """Compile every csrc/*.hip and link libikbo.so, then the probe library. Always rebuilds."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs, LIB)
    if verbose:
        print("built", LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
