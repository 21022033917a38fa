"""Build librax.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Usage: ``python -m prefix_cached_paged_amd.build`` (or ``build()`` from Python). Objects go
to ``prefix_cached_paged_amd/_build/``; the shared library to ``prefix_cached_paged_amd/librax.so``.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librax.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed FP32 VALU ops (v_pk_*_f32) are kept out of generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Loop heads on 64-byte boundaries: without it the hot loops' placement, and their speed
    # (by 1-2%), shifts with the length of whatever code precedes them.
    "-falign-loops=64",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librax)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile every csrc/*.hip and link librax.so. Always recompiles. Returns the library path.

    ``extra_flags`` (e.g. -D overrides of launch-shape constants), ``out`` and ``build_dir``
    let a tuning sweep build variants beside the default library.
    """
    cc = hipcc()
    lib_path = out or LIB
    bdir = build_dir or BUILD
    os.makedirs(bdir, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stdout or r.stderr):
            print(r.stdout + r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib_path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}", file=sys.stderr)
    return lib_path


C_ABI_SRC = os.path.join(ROOT, "tests", "c_abi", "single_key.c")
C_ABI_BIN = os.path.join(ROOT, "tests", "c_abi", "single_key")


def build_c_abi_check(verbose: bool = False) -> str:
    """Compile the plain-C test program against include/librax.h and librax.so (host code only:
    gcc, the HIP runtime API headers and libamdhip64; the library is found next to the package
    at run time)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{os.path.join(ROOT, 'include')}", C_ABI_SRC, "-o", C_ABI_BIN, f"-L{rocm}/lib", "-lamdhip64",
           f"-L{PKG}", "-l:librax.so", f"-Wl,-rpath,{rocm}/lib", "-Wl,-rpath,$ORIGIN/../../prefix_cached_paged_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C test program failed to build:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_ABI_BIN}", file=sys.stderr)
    return C_ABI_BIN


if __name__ == "__main__":
    build(verbose=True)
    build_c_abi_check(verbose=True)
