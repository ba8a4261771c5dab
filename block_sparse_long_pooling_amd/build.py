"""Build libflashprefill.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled on each call (no staleness check), four at a time,
then linked into one shared library next to this file.  build_serial() makes
the debug variant libflashprefill_serial.so, whose kernels fill an LDS tile
buffer only after every read of the previous tile (FP_SERIAL_DMA=1): the race
check compares its results with the pipelined library's bit for bit.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashprefill.so")
SERIAL_LIB = os.path.join(PKG, "libflashprefill_serial.so")
SOURCES = ["fp_abi.hip", "k_pool.hip", "k_quant.hip", "k_select.hip", "k_attn.hip", "k_attn_fp8.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def _build_lib(lib: str, objdir: str, defines, verbose: bool) -> str:
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        out = _run([HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for obj, out in results:
        if verbose and out.strip():
            print(out, file=sys.stderr)
    tmp = lib + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fvisibility=hidden", "-o", tmp,
          *[o for o, _ in results]])
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    return _build_lib(LIB, OBJ, [], verbose)


def build_serial(verbose: bool = False) -> str:
    """The debug variant with serialised LDS tile fills (same entry points)."""
    return _build_lib(SERIAL_LIB, os.path.join(OBJ, "serial"), ["-DFP_SERIAL_DMA=1"], verbose)


ASAN_DIR = os.path.join(PKG, "_build", "asan")


def asan_runtime() -> str:
    """The compiler's shared address-sanitizer runtime (to preload), or ''."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                               text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return ""


def build_host_asan() -> str:
    """A copy of the library whose host code (the C ABI: validation, sizes,
    request tables) is built with the address sanitizer; the kernels are the
    regular objects.  Device code is never instrumented.  Load it with the
    runtime from asan_runtime() preloaded and FLASHPREFILL_LIB pointing at it."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = [os.path.join(OBJ, src.replace(".hip", ".o")) for src in SOURCES if src != "fp_abi.hip"]
    if not all(os.path.exists(o) for o in objs):
        build()
    abi = os.path.join(ASAN_DIR, "fp_abi.o")
    flags = [f for f in CFLAGS if f != "-O3"]
    _run([HIPCC, "-O1", "-g", *flags, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(CSRC, "fp_abi.hip"), "-o", abi])
    lib = os.path.join(ASAN_DIR, "libflashprefill.so")
    clangxx = "/opt/rocm/llvm/bin/clang++"
    _run([clangxx, "-shared", "-fsanitize=address", "-shared-libasan", "-o", lib, abi, *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
