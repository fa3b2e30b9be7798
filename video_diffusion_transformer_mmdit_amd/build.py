"""Build libmmdit.so (all HIP sources for gfx950) in-tree.

    python -m video_diffusion_transformer_mmdit_amd.build

Every source under csrc/ is compiled with hipcc into _build/ and linked into
video_diffusion_transformer_mmdit_amd/libmmdit.so.  Packed fp32 VALU instructions are
disabled for the device code.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmmdit.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "block.hip", "gemm.hip", "joint_attention.hip", "modulate_ln.hip", "quant.hip",
           "attn8_quant.hip", "joint_attention_8bit.hip",
           "modulation.hip", "qk_norm_rope.hip"]

CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-file flags.  The attention kernels never produce or consume NaN on valid input (masked
# scores are -inf, never NaN), so IEEE NaN canonicalisation of every max is dropped there.
FILE_FLAGS = {"joint_attention.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *CFLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # a kernel whose host stub the compiler dropped (a deferred host-side diagnostic) links
    # fine and only fails when loaded: load it here so the build fails instead
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:])
