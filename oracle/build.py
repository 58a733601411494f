"""Build the CPU oracle (plain C, fp64) into oracle/liboracle.so with gcc.

Test infrastructure only: see oracle/__init__.py.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every product and sum rounds as written.
# No -ffast-math: the compiler may not reassociate the ascending-index sums.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


# The sanitizer build (ASan + UBSan, aborting on the first report) uses ROCm's clang,
# whose runtime the host part of libpfgemm.so is sanitized with too, so that both
# libraries run in one process under one preloaded runtime.
SAN_CC = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def build(force=True, sanitize=False):
    """Compile the oracle; returns the library path. sanitize: ASan + UBSan build
    (to be loaded with the clang ASan runtime preloaded; see tests/sanitize_run.py)."""
    if not force and not sanitize and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    if sanitize:
        cmd = [SAN_CC, *CFLAGS, "-fopenmp=libgomp", *SAN_FLAGS, SRC, "-o", tmp, "-lm"]
        cmd.remove("-fopenmp")
    else:
        cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(sanitize="--sanitize" in sys.argv))
