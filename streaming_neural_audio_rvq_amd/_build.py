"""Build of the gfx950 HIP library ``libsnrvq.so`` (in-tree, next to this file).

Every source is compiled with hipcc for gfx950 only, in parallel, into
``_build/`` and linked into one shared library with a plain C ABI
(``include/snrvq.h``).

``build_hostsan()`` links a second copy, ``libsnrvq_hostsan.so``, whose host
code (``api.cpp``: argument checks, batch assembly, planning, graphs) is
built with AddressSanitizer and UndefinedBehaviorSanitizer; the device code
is the same objects as in ``libsnrvq.so`` (no GPU sanitizer).  A process
loads it with the ASan runtime preloaded (``asan_runtime()``) and selects it
with ``SNRVQ_LIBRARY``.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsnrvq.so")
LIB_HOSTSAN = os.path.join(HERE, "libsnrvq_hostsan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "kernels_conv.hip", "kernels_misc.hip", "kernels_tf.hip",
           "kernels_stage.hip"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-I" + INCLUDE, "-I" + CSRC,
          # no packed-fp32 instructions anywhere in device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# host-only sanitizers: each -fsanitize= applies to the host pass alone
HOSTSAN = ["-g", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, extra=(), obj=None) -> str:
    obj = obj or os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


LIB_PROBES = os.path.join(HERE, "libsnrvq_probes.so")


def build_probes(verbose: bool = False) -> str:
    """libsnrvq_probes.so: the micro-benchmarks of probes/ceilings.hip
    (include/snrvq_probes.h), a library of their own."""
    os.makedirs(BUILD, exist_ok=True)
    src = os.path.join(HERE, "probes", "ceilings.hip")
    tmp = LIB_PROBES + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceilings.hip:\n{r.stderr}")
    os.replace(tmp, LIB_PROBES)
    if verbose:
        print("built", LIB_PROBES)
    return LIB_PROBES


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found: " + (r.stderr or path))
    return path


def build_hostsan(verbose: bool = False) -> str:
    """libsnrvq_hostsan.so: api.cpp with host ASan + UBSan, the kernels'
    objects of the last build() (built first if missing)."""
    kobjs = [os.path.join(BUILD, src + ".o") for src in SOURCES if src != "api.cpp"]
    if not all(os.path.exists(o) for o in kobjs):
        build()
    obj = _compile("api.cpp", HOSTSAN, os.path.join(BUILD, "api.cpp.hostsan.o"))
    tmp = LIB_HOSTSAN + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, obj, *kobjs,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_HOSTSAN)
    if verbose:
        print("built", LIB_HOSTSAN)
    return LIB_HOSTSAN


if __name__ == "__main__":
    build(verbose=True)
    build_hostsan(verbose=True)
    build_probes(verbose=True)
