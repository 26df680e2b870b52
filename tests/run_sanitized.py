"""Run the CPU test tier against builds with AddressSanitizer and
UndefinedBehaviorSanitizer in their host code.

    python tests/run_sanitized.py [extra pytest args]

Builds, under _build/sanitize/:
  * liboracle.so: oracle/oracle.cpp with clang, -fsanitize=address,undefined
    (OpenMP through GCC's runtime, as the plain g++ builds of the mutant
    tests use);
  * libpw.so: the library with the host code of pw_api.cpp and noalloc.hip
    (argument validation, planning, workspace layout, launch set-up)
    instrumented the same way (-Xarch_host: device code is built as usual),
    linked with the other objects of the normal build.
Then runs `pytest tests -m "not gpu"` with clang's sanitizer runtime
preloaded (the Python interpreter is not instrumented), the two builds
selected through PW_LIBRARY and PW_ORACLE_LIBRARY, leak checking off (the
interpreter keeps its allocations) and any report fatal. Exits with
pytest's status. Needs a normal build first (python -m
lazy_score_matrix_amd.build), whose device objects it reuses.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from lazy_score_matrix_amd import build as pwbuild  # noqa: E402

OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
HOST_SOURCES = ("pw_api.cpp", "noalloc.hip")


def runtime():
    libs = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang's AddressSanitizer runtime is not installed under %s" % LLVM)
    return libs[0]


def build_oracle():
    out = os.path.join(OUT, "liboracle.so")
    cmd = [os.path.join(LLVM, "bin", "clang++"), "-O1", "-std=c++17", "-fPIC", "-shared", "-fopenmp=libgomp"] + SAN + \
          [os.path.join(ROOT, "oracle", "oracle.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def build_library():
    tag = pwbuild._headers_digest()
    objs = []
    for src in pwbuild.sources():
        name = os.path.basename(src)
        if name in HOST_SOURCES:
            obj = os.path.join(OUT, name + ".o")
            extra = pwbuild.KERNEL_FLAGS if src.endswith(".hip") else []
            host = [f for flag in SAN for f in ("-Xarch_host", flag)]
            subprocess.run([pwbuild.HIPCC] + pwbuild.FLAGS + extra + host + ["-c", src, "-o", obj], check=True)
        else:
            obj = os.path.join(pwbuild.BUILD, "%s.%s.o" % (name, tag))
            if not os.path.exists(obj):
                raise SystemExit("missing %s: run `python -m lazy_score_matrix_amd.build` first" % obj)
        objs.append(obj)
    out = os.path.join(OUT, "libpw.so")
    subprocess.run([pwbuild.HIPCC, "-shared", "-fPIC", "--offload-arch=" + pwbuild.ARCH, "-o", out] + objs, check=True)
    return out


def main():
    os.makedirs(OUT, exist_ok=True)
    env = dict(os.environ)
    logs = os.path.join(OUT, "report")
    for f in glob.glob(logs + ".*"):
        os.remove(f)
    # Reports go to files: a sanitizer stops the process at once, and pytest
    # would lose what it wrote into its output capture.
    env.update({
        "PW_ORACLE_LIBRARY": build_oracle(),
        "PW_LIBRARY": build_library(),
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:log_path=" + logs,
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:log_path=" + logs,
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-p", "no:cacheprovider"]
    rc = subprocess.run(cmd + sys.argv[1:], env=env, cwd=ROOT).returncode
    for f in sorted(glob.glob(logs + ".*")):
        print("==== sanitizer report %s" % f)
        print(open(f).read())
        rc = rc or 1
    sys.exit(rc)


if __name__ == "__main__":
    main()
