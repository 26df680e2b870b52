"""Build libpw.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into lazy_score_matrix_amd/libpw.so. Run as
``python -m lazy_score_matrix_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpw.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed FP32 instructions are kept out of every code object.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


# Device code: NaN scores are unsupported (include/pw.h), so kernels are built
# without NaN semantics; min/max then need no operand canonicalisation. IEEE
# mode stays on: a kernel built without it cannot inline the device library
# (work-item ids, float64 exp/log), and every kernel would call those out of
# line. Host validation (pw_api.cpp) keeps full NaN handling.
KERNEL_FLAGS = ["-fno-honor-nans"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _headers_digest():
    h = hashlib.sha1()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith(".h"):
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(f.encode() + fh.read())
    h.update(" ".join(FLAGS + KERNEL_FLAGS).encode())
    return h.hexdigest()[:16]


def _compile(src, obj, verbose):
    extra = KERNEL_FLAGS if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (os.path.basename(src), r.stdout, r.stderr))
    return obj


def build(jobs: int | None = None, force: bool = False, verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libpw.so. Returns its path.

    Objects are rebuilt when their source or any header changed; the link
    always runs, so the library is fresh after every call.
    """
    os.makedirs(BUILD, exist_ok=True)
    tag = _headers_digest()
    jobs = jobs or min(16, os.cpu_count() or 4)
    todo, objs = [], []
    for src in sources():
        obj = os.path.join(BUILD, "%s.%s.o" % (os.path.basename(src), tag))
        objs.append(obj)
        if force or not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
            todo.append((src, obj))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), todo))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose="-v" in sys.argv))
