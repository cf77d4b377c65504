"""Build libmx.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Runs without a GPU: hipcc cross-compiles the device code. Objects go to
_build/ at the repository root; the library is written next to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmx.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mx_api.cpp", "quantize.hip", "dequantize.hip", "gemm_mx.hip", "gemm_mxfp4.hip", "gemm_bf16x.hip", "gemm_bf16x_large.hip",
           "gemm_w4a16.hip", "gemm_mbs.hip", "pack.hip"]

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
# -ffp-contract=off: every fp32 step of the NVFP4 quantizer rounds once.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


# Per-source flags. gemm_mbs.hip: the MFMA partial sums feed vector-ALU
# arithmetic, so select the MFMA forms that write VGPRs (the default puts them
# in AGPRs and adds one v_accvgpr_read per element).
EXTRA = {"gemm_mbs.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    """Compile every source and link libmx.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    build_calib()
    return OUT


CALIB_OUT = os.path.join(HERE, "libmx_calib.so")


def build_calib():
    """libmx_calib.so: the matrix-instruction ceiling of include/mx_calib.h
    (measurement only; libmx.so does not use it)."""
    obj, err = _compile("calib.hip")
    tmp = CALIB_OUT + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, CALIB_OUT)
    return CALIB_OUT


if __name__ == "__main__":
    print(build(verbose=True))


SAN_OUT = os.path.join(BUILD, "libmx_hostsan.so")


def build_host_sanitized():
    """libmx with its host code (the C ABI: argument checks, dispatch, error
    mapping) compiled by g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernels' objects from build().
    For CPU tests of the ABI only (loaded in a child process that preloads the
    ASan runtime); written to _build/, never used by the GPU path."""
    if not all(os.path.exists(os.path.join(BUILD, src + ".o")) for src in SOURCES):
        build()
    obj = os.path.join(BUILD, "mx_api_hostsan.o")
    cxx = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-c", os.path.join(CSRC, "mx_api.cpp"), "-o", obj]
    r = subprocess.run(cxx, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed for mx_api.cpp:\n" + r.stderr)
    kernels = [os.path.join(BUILD, src + ".o") for src in SOURCES if src != "mx_api.cpp"]
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", obj, *kernels,
            "-lasan", "-lubsan", "-o", SAN_OUT]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return SAN_OUT
