"""Build the gfx950 HIP library in-tree: softmax_attention_paged_amd/libattn_mi355x.so.

Every source under csrc/ is compiled with hipcc for gfx950 only, then linked
into one shared library exporting the C ABI declared in include/attn.h. The
benchmark's ceiling kernels (ceilings/ceilings.hip) go into a second object,
libattn_ceilings.so.

    python -m softmax_attention_paged_amd.build [-v]
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# The benchmark's ceiling kernels (a streaming read, an MFMA loop): their own
# shared object, not part of the attention library.
CEIL_SRC = os.path.join(PKG_DIR, "ceilings", "ceilings.hip")
CEIL_PATH = os.path.join(PKG_DIR, "libattn_ceilings.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Wall", "-Wextra", "-Wno-unused-parameter", "-Werror",
    # Let the compiler emit no packed-FP32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = os.environ.get("ATTN_HIPCC_EXTRA", "").split()
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link the shared library.
    Always rebuilds. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(LIB_PATH, objs, verbose)
    _link(CEIL_PATH, [_compile(CEIL_SRC, verbose)], verbose)
    return LIB_PATH


def _link(path: str, objs: list[str], verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
