"""Build libfattn.so (HIP kernels + C-ABI host code) for gfx950, in-tree.

Every source is compiled by hipcc for --offload-arch=gfx950 into
``tiled_attention_fattn_amd/_build/`` and linked into
``tiled_attention_fattn_amd/libfattn.so``. Packed-FP32 instruction selection
is disabled for all device code. MFMA results are selected into ordinary
VGPRs where registers allow (the backend's VGPR form): a kernel that runs the
softmax on an MFMA accumulator then reads it directly instead of copying it
out of the accumulation registers first. Of the kernels here only the
d = 128 dK/dV kernels, which need the accumulation registers, compile
differently (a third fewer register copies in their loop, 2.5-4% on the
backward, bit-identical results).

    python -m tiled_attention_fattn_amd.build [-v]
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfattn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["fattn_host.cpp", "fwd_bf16.hip", "bwd_bf16.hip", "fwd_fp8.hip", "static_ws.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", CSRC, "-I", INCLUDE, "-Wall", "-Wno-unused-result"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is noise.
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return obj


def build(verbose=False):
    """Compile every source and link libfattn.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # Every kernel's host stub must be defined: a host-pass problem in a kernel
    # body can drop a stub silently and leave an undefined symbol behind.
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
