"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Rebuilds the oracle and the host validation of libpfgemm.so (pf_api.cpp) with
-fsanitize=address,undefined, runs `pytest -m "not gpu"` with the clang ASan runtime
preloaded (any report aborts the run), then rebuilds both libraries without
sanitizers and exits with pytest's status.

    python tests/sanitize_run.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    from oracle import build as oracle_build
    from quantized_weight_prefill_gguf_amd import build as pf_build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang ASan runtime not found")
    oracle_build.build(sanitize=True)
    pf_build.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    try:
        rc = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-m", "not gpu",
                             "-p", "no:cacheprovider", *sys.argv[1:]], cwd=ROOT, env=env).returncode
    finally:
        oracle_build.build()
        pf_build.build()
    sys.exit(rc)


if __name__ == "__main__":
    main()
