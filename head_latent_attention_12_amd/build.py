"""Compile the HIP library (libmla.so) for gfx950 in place.

Usage: python -m head_latent_attention_12_amd.build
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRC = os.path.join(CSRC, "mla.hip")
SRC_FP8 = os.path.join(CSRC, "decode_fp8.hip")
SRC_FOLD = os.path.join(CSRC, "fold.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# mla.hip: MFMA accumulators in VGPR form, which lets the allocator keep the
# bf16 decode kernel's 32x512 fp32 accumulator block (AGPR operands of its asm
# blocks) and its q fragments without scratch.  decode_fp8.hip is compiler
# scheduled and needs the default form (accumulators in AGPRs).
MLA_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
HIPCC_FLAGS = COMMON_FLAGS + MLA_FLAGS  # (kept for callers that compile mla.hip alone)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the library's
# argument checks and planning code (the device code is built as usual): each
# -fsanitize= applies to the host pass only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, extra=(), sanitize: bool = False, out: str | None = None) -> str:
    """Compile the translation units (each with its own flags) and link them
    into ``out`` (default: the package's libmla.so).  ``sanitize``: host code
    built with ASan and UBSan (load it with the clang ASan runtime preloaded)."""
    lib = out or LIB
    tmp = lib + ".tmp"
    san = SANITIZE_HOST if sanitize else []
    objs = []
    for src, flags in ((SRC, COMMON_FLAGS + MLA_FLAGS), (SRC_FP8, COMMON_FLAGS), (SRC_FOLD, COMMON_FLAGS)):
        obj = os.path.join(os.path.dirname(lib), os.path.basename(src) + (".san.o" if sanitize else ".o"))
        _run([hipcc(), *flags, *san, *extra, "-I", INCLUDE, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    try:
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, "-o", tmp], verbose)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    _check_kernel_stubs(tmp)
    os.replace(tmp, lib)
    return lib


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc's host compiler (to preload)."""
    res = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found next to hipcc")
    return path


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
