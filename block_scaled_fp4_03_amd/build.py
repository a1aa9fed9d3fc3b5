"""Build libfp4.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m block_scaled_fp4_03_amd.build

Each translation unit is compiled separately (in parallel) into _build/, then
linked into block_scaled_fp4_03_amd/libfp4.so.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libfp4.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "quantize.hip", "gemm.hip", "gemm_w4a8.hip", "gemv_nv.hip", "gemv_nv_blocksum.hip",
           "gemv_nv_dot.hip"]

# -ffp-contract=off: no silent a*b+c fusion (the quantiser must round exactly
# like the IEEE definition).  The packed-FP32 feature is switched off for the
# device code: hipcc forms v_pk_* FP32 ops from scalar code otherwise.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


def build_sanitized(verbose=False):
    """A host-sanitized copy of the library for the CPU test of the ABI's
    validation paths: abi.cpp compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host code only (each sanitizer flag
    behind -Xarch_host; the kernels are the normal objects of build()).  The
    sanitizer runtime is not linked in: a process that loads this library
    preloads clang's libclang_rt.asan (see tests/test_sanitizers.py).
    Returns the library's path."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, s + ".o")) for s in SOURCES):
        build()
    san_dir = os.path.join(BUILD_DIR, "sanitize")
    os.makedirs(san_dir, exist_ok=True)
    obj = os.path.join(san_dir, "abi.cpp.o")
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
    cmd = [_hipcc(), "-x", "hip"] + COMMON + host + ["-c", os.path.join(CSRC, "abi.cpp"), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized abi.cpp failed:\n" + res.stdout + res.stderr)
    out = os.path.join(san_dir, "libfp4_san.so")
    objs = [obj] + [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s != "abi.cpp"]
    res = subprocess.run([_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", out] + objs,
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + res.stdout + res.stderr)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
