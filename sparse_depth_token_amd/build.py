"""Build the HIP library libxmod.so in-tree for gfx950 (hipcc cross-compiles without a GPU).

Usage: python -m sparse_depth_token_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libxmod.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["route.hip", "rows.hip", "rows_bwd.hip", "gemm.hip", "attention.hip",
           "attention_bwd.hip", "probe.hip",
           "xmod_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-munsafe-fp-atomics",
    # packed-fp32 instruction forms stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Host AddressSanitizer on the library's host code only (argument checks, workspace planning,
# launch set-up); the device code is built as in the product. Each sanitizer flag sits right
# after -Xarch_host so that it reaches the host compilation alone.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-shared-libasan"]


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose: bool = False, out: str = OUT, build_dir: str = BUILD_DIR,
          host_asan: bool = False) -> str:
    """Compile every source and link the library (libxmod.so in the package unless `out` says
    otherwise); always rebuilds. host_asan: host code under AddressSanitizer (load the result
    with the sanitizer's runtime preloaded). Returns the library path."""
    os.makedirs(build_dir, exist_ok=True)
    extra = ASAN_FLAGS if host_asan else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp,
                        *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # every internal symbol must be defined (a kernel whose host stub was dropped shows up here)
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "xmod" in l]
    if missing:
        raise RuntimeError("undefined library symbols after link: " + ", ".join(missing[:5]))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
