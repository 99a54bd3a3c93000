"""Build libsplitkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m block_sparse_cross_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsplitkv.so")
SOURCES = ["api.hip", "anchors.hip", "plan.hip", "merge.hip", "attn_fwd.hip", "attn_bwd.hip",
           "gemm.hip"]
# The matrix-core ceiling loop (bench.py's context), a library of its own.
CEILING_LIB = os.path.join(HERE, "libsplitkv_ceiling.so")
CEILING_SOURCES = ["mfma_ceiling.hip"]
ARCH = os.environ.get("SPLITKV_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-munsafe-fp-atomics",
    # packed fp32 ops disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]
# Per-file code generation choices. The backward's dK/dV kernel holds its dK, dV
# accumulators in AGPRs; the matrix products of the scores then default to the
# AGPR form too, and every score is copied back before the softmax. The VGPR
# form keeps the scores where the vector ALU reads them (measured: dK/dV about
# 2% faster, no change to the arithmetic).
EXTRA_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


# Host code (the C ABI's validation and launch setup) checked by Address- and
# UndefinedBehaviorSanitizer; device code is built as usual. Such a library
# runs with clang's ASan runtime preloaded (see host_asan_runtime()).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer"]


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + EXTRA_FLAGS.get(src, []) + list(extra) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out: str, extra=()) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + list(extra) + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False, host_sanitize_to: str = "") -> str:
    """Compile and link the library (in-tree) and the ceiling library beside it,
    or, with host_sanitize_to, only a copy of the library whose host code
    carries the sanitizers, at that path."""
    out = host_sanitize_to or LIB
    objdir = os.path.join(os.path.dirname(out), "_obj_san") if host_sanitize_to else OBJDIR
    extra = HOST_SANITIZE if host_sanitize_to else []
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES if host_sanitize_to else SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda src: _compile(src, objdir, extra), srcs)))
    _link([objs[x] for x in SOURCES], out,
          ["-Xarch_host", "-shared-libsan"] if host_sanitize_to else [])
    if not host_sanitize_to:
        _link([objs[x] for x in CEILING_SOURCES], CEILING_LIB)
    if verbose:
        print("built", out)
    return out


def host_asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime (to preload for a library built
    with host_sanitize_to)."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
