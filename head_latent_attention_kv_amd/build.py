"""Compile the HIP kernels and the C ABI into libmla_amd.so (gfx950), in-tree.

    python -m head_latent_attention_kv_amd.build [-v] [--variant release|debug|hostsan|all]

Each source under csrc/ is compiled with hipcc for --offload-arch=gfx950 into
_build/<variant>/, then linked into head_latent_attention_kv_amd/:
  release  libmla_amd.so        the library
  debug    libmla_amd_debug.so  the same with MLA_DEBUG_CHECKS: decode, prefill and
                                cache-write calls copy their index arrays to the host
                                (synchronising) and refuse out-of-range ones
  hostsan  libmla_amd_hostsan.so  MLA_DEBUG_CHECKS, and the host code built with
                                AddressSanitizer and UndefinedBehaviorSanitizer (the
                                kernels as in release): for checking the argument
                                validation on the CPU
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
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]

VARIANTS = {
    "release": dict(lib="libmla_amd.so", flags=["-O3"], link=[]),
    "debug": dict(lib="libmla_amd_debug.so", flags=["-O3", "-DMLA_DEBUG_CHECKS"], link=[]),
    # sanitizers on the host pass only (-Xarch_host before each one); the kernels
    # are compiled as in the release build
    "hostsan": dict(lib="libmla_amd_hostsan.so",
                    flags=["-O1", "-g", "-fno-omit-frame-pointer", "-DMLA_DEBUG_CHECKS",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"],
                    link=["-shared-libsan",
                          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]),
}
LIB = os.path.join(PKG, VARIANTS["release"]["lib"])


def lib_path(variant: str = "release") -> str:
    return os.path.join(PKG, VARIANTS[variant]["lib"])


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, variant: str, verbose: bool) -> str:
    out_dir = os.path.join(BUILD, variant)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *VARIANTS[variant]["flags"], *COMMON, "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, variant: str = "release") -> str:
    """Compile and link one variant; returns the library's path."""
    v = VARIANTS[variant]
    os.makedirs(os.path.join(BUILD, variant), exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, variant, verbose), srcs))
    out = os.path.join(PKG, v["lib"])
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *v["link"], *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    which = "release"
    if "--variant" in sys.argv:
        which = sys.argv[sys.argv.index("--variant") + 1]
    for name in (VARIANTS if which == "all" else [which]):
        print(build(verbose="-v" in sys.argv, variant=name))
