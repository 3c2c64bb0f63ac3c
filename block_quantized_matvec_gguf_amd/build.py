"""Build libqmv.so (the HIP library behind include/qmv.h) for gfx950 with
hipcc. Sources compile in parallel into _build/, then link in place next to
this file. Run as ``python -m block_quantized_matvec_gguf_amd.build``."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmv.so")
SOURCES = ["qmv_api.cpp", "qmv_gemv.hip", "qmv_gemv_t.hip", "qmv_simple.hip", "qmv_mfma.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            # no packed-FP32 VALU instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument"]


# Host code of this build is instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (device code is built as usual); the CPU tests
# exercise its argument validation and planning with the sanitizer runtime
# preloaded. It is never loaded on a GPU.
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libqmv_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(cc, src, outdir, extra, verbose):
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [cc] + common_flags() + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out:
        print(out)
    return obj


def _link(cc, objs, lib, extra):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH] + extra + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False, sanitized: bool = True) -> str:
    """Build libqmv.so and, with sanitized=True, the host-sanitizer build
    next to the objects (both in parallel)."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(SAN_BUILD, exist_ok=True)
    cc = hipcc()
    jobs = [(src, BUILD, []) for src in SOURCES]
    if sanitized:
        jobs += [(src, SAN_BUILD, SAN_FLAGS) for src in SOURCES]
    # the slowest sources first
    jobs.sort(key=lambda j: os.path.getsize(os.path.join(CSRC, j[0])), reverse=True)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda j: (j[1], _compile(cc, j[0], j[1], j[2], verbose)), jobs))
    _link(cc, [o for d, o in objs if d == BUILD], LIB, [])
    if sanitized:
        _link(cc, [o for d, o in objs if d == SAN_BUILD], SAN_LIB,
              ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"])
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
