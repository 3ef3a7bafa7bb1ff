"""Build the HIP library in-tree: packed_cache_decode_amd/libtq_mi355x.so.

    python -m packed_cache_decode_amd.build_lib

Compiles for gfx950 only.  The store translation unit is built without
floating-point contraction (its bytes must be reproducible bit for bit);
packed fp32 instructions are disabled for all device code.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq_mi355x.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
SOURCES = [
    ("tq_host.cpp", []),
    ("tq_store.hip", ["-ffp-contract=off"]),
    ("tq_store_quad.hip", ["-ffp-contract=off"]),
    ("tq_decode.hip", []),
    ("tq_decode_mfma.hip", ["-fno-honor-nans"]),
    ("tq_dequant.hip", []),
    ("tq_probe.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r.stdout


def build(verbose=False):
    """Compile every translation unit (in parallel) and link the library."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    cmds, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC, *COMMON, *lang, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as pool:
        outs = list(pool.map(_run, cmds))
    if verbose:
        for out in outs:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libtq_mi355x_asan.so")


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime (None if absent)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_host_asan():
    """The library with its host code (tq_host.cpp: codebook solvers, tables,
    planning, argument checks) built with AddressSanitizer, device code as in
    build(); for CPU checks of the host logic (load it in a process started
    with the sanitizer runtime preloaded).  Needs build()'s objects."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if src == "tq_host.cpp":
            obj = os.path.join(ASAN_DIR, "tq_host.o")
            # host pass only: each sanitizer flag behind -Xarch_host
            _run([HIPCC, *COMMON, "-x", "hip", *extra, "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, src), "-o", obj])
        elif not os.path.exists(obj):
            raise RuntimeError(f"{obj} missing: run build() first")
        objs.append(obj)
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-shared-libasan", "-o", ASAN_LIB, *objs])
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
