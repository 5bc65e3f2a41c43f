"""Build libbdfp4.so (HIP, gfx950) in-tree with hipcc.

    python -m fp4_kv_cache_nvfp4_amd.build [--sanitize]

Compiles every source under csrc/ to an object and links the shared library
fp4_kv_cache_nvfp4_amd/lib/libbdfp4.so. Flags that matter for results:
-ffp-contract=off (no fused multiply-add where the codecs need separate
roundings), correctly rounded float32 division, and packed-FP32 instructions
disabled (the v_pk_*_f32 forms are kept out of every kernel). With
--sanitize it builds lib/libbdfp4_san.so instead, its host API under ASan and
UBSan (see build_sanitized).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libbdfp4.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["api.cpp", "writer.hip", "decode.hip", "bf16_decode.hip", "stream.hip", "calib.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI
# layer (each -fsanitize= after -Xarch_host: device code is built as usual).
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_LIB = os.path.join(LIBDIR, "libbdfp4_san.so")


def build_sanitized(verbose: bool = True) -> str:
    """lib/libbdfp4_san.so: the library with its host API (api.cpp: every
    recipe, shape, pointer and workspace check, the plan and the tau choice)
    compiled under ASan and UBSan, linked with the regular device objects.
    Load it after the sanitizer runtime (LD_PRELOAD of the clang ASan
    runtime); the CPU test of the host ABI runs this way."""
    if not all(os.path.exists(os.path.join(BUILD, s + ".o")) for s in SOURCES):
        build(verbose=False)
    obj = os.path.join(BUILD, "api.cpp.san.o")
    cmd = [hipcc(), *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized api.cpp:\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "api.cpp"]
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized library needs."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if c and os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            p = r.stdout.strip()
            if r.returncode == 0 and os.path.exists(p):
                return p
    raise RuntimeError("clang ASan runtime not found")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--sanitize":
        build_sanitized()
    else:
        build()
