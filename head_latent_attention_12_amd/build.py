"""Compile the HIP library (libmla.so) for gfx950 in place.

Usage: python -m head_latent_attention_12_amd.build
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mla.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPR form: lets the allocator keep the decode
    # kernel's 32x512 fp32 accumulator block and its q fragments without scratch
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    _check_kernel_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_kernel_stubs(path: str) -> None:
    """Fail if a kernel's host launch stub is referenced but not defined (the
    library would then not load): the host pass can drop the stub of a kernel
    template instance without an error."""
    nm = shutil.which("nm")
    if nm is None:
        return
    res = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True)
    missing = [line.split()[-1] for line in res.stdout.splitlines() if "__device_stub__" in line]
    if missing:
        raise RuntimeError(f"{path}: kernel launch stubs missing: {missing}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
