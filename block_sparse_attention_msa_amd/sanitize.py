"""AddressSanitizer + UndefinedBehaviorSanitizer run of the host code.

Builds instrumented copies of the HIP library (its host code: the C-ABI
validation, workspace layout and launch orchestration; device code is built as
usual) and of the fp64 oracle under _build/sanitize/, then runs the CPU test
suite (-m "not gpu": oracle pins, parity-rule checks, C-ABI validation) against
them with clang's sanitizer runtime preloaded into the interpreter.  Any report
fails the run (UBSan findings abort; leak detection is off because the
interpreter itself keeps its allocations until exit).

    python -m block_sparse_attention_msa_amd.sanitize [extra pytest args]

Exit status: pytest's.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as hip_build

OUT = os.path.join(hip_build.ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
# host-side instrumentation only: each option reaches the host compilation
HOST_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
            "-shared-libasan", "-g"]


def _host(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def asan_runtime() -> str:
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")
    return libs[-1]


def build() -> dict:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for name in hip_build.SOURCES:
        obj = os.path.join(OUT, name + ".o")
        cmd = ([hip_build.HIPCC] + hip_build.FLAGS + hip_build.FILE_FLAGS.get(name, []) + _host(HOST_SAN) +
               ["-c", "-x", "hip", os.path.join(hip_build.CSRC, name), "-o", obj])
        subprocess.check_call(cmd)
        objs.append(obj)
    lib = os.path.join(OUT, "libmsa.so")
    subprocess.check_call([hip_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + _host(HOST_SAN) + objs +
                          ["-o", lib])
    ceiling = os.path.join(OUT, "libmsa_ceiling.so")
    subprocess.check_call([hip_build.HIPCC] + hip_build.FLAGS + _host(HOST_SAN) +
                          ["-shared", "-x", "hip", os.path.join(hip_build.CSRC, hip_build.CEILING_SOURCE), "-o",
                           ceiling])
    orc = os.path.join(OUT, "libmsa_oracle.so")
    src = os.path.join(hip_build.ROOT, "oracle", "msa_oracle.c")
    subprocess.check_call([CLANG, "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"] + HOST_SAN +
                          [src, "-o", orc, "-lm"])
    return {"MSA_LIB_PATH": lib, "MSA_ORACLE_LIB": orc}


def main(argv) -> int:
    env = dict(os.environ)
    env.update(build())
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(hip_build.ROOT, "tests"), "-q", "-m", "not gpu", "-x"] + argv
    print("sanitized libraries:", env["MSA_LIB_PATH"], env["MSA_ORACLE_LIB"], flush=True)
    return subprocess.call(cmd, env=env, cwd=hip_build.ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
