"""Builds libhysparse.so (all HIP sources, gfx950) in the package directory.

    python -m long_context_split_amd.build [--jobs N]

Each source is compiled to an object with hipcc in parallel, then linked into
one shared library next to this file.  Always rebuilds (cheap objects are
reused only when their source and flags are unchanged).
"""

import concurrent.futures
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhysparse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["hs_attn.hip", "hs_wave.hip", "hs_rows.hip", "hs_gather.hip", "hs_select.hip", "hs_bridge.hip", "hs_append.hip", "hs_swa.hip", "hs_filter.hip", "hs_probe.hip", "hs_api.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def _digest(src):
    h = hashlib.sha256()
    h.update(" ".join(FLAGS).encode())
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hpp", ".h")):
            h.update(open(os.path.join(CSRC, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "hysparse.h"), "rb").read())
    h.update(open(os.path.join(CSRC, src), "rb").read())
    return h.hexdigest()[:16]


def _compile(src, verbose):
    obj = os.path.join(OBJ, src.replace(".hip", ".o"))
    stamp = obj + ".sha"
    dig = _digest(src)
    if os.path.exists(obj) and os.path.exists(stamp) and open(stamp).read() == dig:
        return obj
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    open(stamp, "w").write(dig)
    return obj


def build(verbose=False, jobs=None, force=False):
    os.makedirs(OBJ, exist_ok=True)
    if force:
        for f in os.listdir(OBJ):
            os.remove(os.path.join(OBJ, f))
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, flush=True)
    return LIB


# Host-code sanitizers for the C ABI layer: hs_api.hip (argument checks, planning, launch
# sequencing) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host side
# only (each -fsanitize= after -Xarch_host; the device code is built as usual) and linked with the
# regular objects of the kernel sources.  Loaded with the clang ASan runtime preloaded.
SANITIZED_LIB = os.path.join(OBJ, "libhysparse_sanitized.so")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime():
    """Path of the clang AddressSanitizer runtime of this ROCm toolchain, or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized(verbose=False):
    build(verbose=verbose)                                   # the kernel objects
    obj = os.path.join(OBJ, "hs_api_sanitized.o")
    cmd = [HIPCC] + FLAGS + SANITIZE + ["-c", os.path.join(CSRC, "hs_api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized hs_api.hip:\n" + r.stderr)
    objs = [os.path.join(OBJ, f.replace(".hip", ".o")) for f in SOURCES if f != "hs_api.hip"] + [obj]
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", SANITIZED_LIB] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        build(verbose=True, force="--force" in sys.argv)
