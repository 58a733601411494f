"""Build libpfgemm.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m quantized_weight_prefill_gguf_amd.build
"""
import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpfgemm.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["pf_api.cpp", "pf_dequant.hip", "pf_gemm_f32.hip", "pf_gemm_f16.hip", "pf_gemv.hip",
           "pf_rmsnorm.hip", "pf_argmax.hip", "pf_noalloc.hip", "pf_xq.hip", "pf_probe.hip",
           "pf_gemv_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# gfx950 only. Packed fp32 instructions are switched off for device code (the
# host pass warns that it does not know the feature; that is harmless).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# Sanitizer switch for the host-side argument validation (pf_api.cpp, the C ABI's
# checks that run before any HIP call): ASan + UBSan on its host code, each
# -fsanitize directly after -Xarch_host so that no device code is built with it.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_SOURCES = ("pf_api.cpp",)


def _compile(src, sanitize=False):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    san = SAN_HOST if sanitize and src in SAN_SOURCES else []
    cmd = [HIPCC, *FLAGS, *san, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(sanitize=False):
    """Compile every source and link libpfgemm.so; returns its path. sanitize: the
    host validation in pf_api.cpp built with ASan + UBSan (load the library with the
    clang ASan runtime preloaded; see tests/sanitize_run.py)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(sanitize="--sanitize" in sys.argv))
