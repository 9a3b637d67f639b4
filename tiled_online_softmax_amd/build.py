"""Build libfa.so (the HIP library) in-tree with hipcc for gfx950.

Usage: python -m tiled_online_softmax_amd.build [--verbose] [--sanitize OUT.so]
Every source under csrc/ is compiled to an object and the objects are
linked into tiled_online_softmax_amd/libfa.so. Compilation always runs (no
staleness check), so calling this after editing a source is enough.

--sanitize OUT.so builds the same library with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (each -fsanitize follows
-Xarch_host; the GPU code is compiled exactly as in the normal build) and
writes it to OUT.so instead. The sanitizer runtime is not linked in: load
the library with FA_LIBRARY=OUT.so into a process that has the clang ASan
runtime (sanitizer_runtime(), which also carries the UBSan handlers)
preloaded. It is for the host-side argument checks, which run without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-variable", "-Wno-unused-parameter",
    # no packed-FP32 VALU instructions anywhere (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfa)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, objdir, extra, verbose):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + extra + ["-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


# Host-only sanitizer flags: every -fsanitize directly after -Xarch_host.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-O1", "-g"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime matching hipcc (it also carries the UBSan handlers)."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    if not os.path.isdir(root):
        root = "/opt/rocm/llvm/lib/clang"
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("clang ASan runtime not found")


def build(verbose: bool = False, extra=(), out: str = LIB, sanitize: bool = False) -> str:
    extra = list(extra) + (SANITIZE_FLAGS if sanitize else [])
    with tempfile.TemporaryDirectory(prefix="libfa_build_") as td:
        srcs = sources()
        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            objs = list(ex.map(lambda s: _compile(s, td, extra, verbose), srcs))
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build(verbose="--verbose" in sys.argv, out=os.path.abspath(sys.argv[sys.argv.index("--sanitize") + 1]),
                    sanitize=True))
    else:
        print(build(verbose="--verbose" in sys.argv))
