"""Build libpa.so (HIP for gfx950 + the host allocator) in the package directory.

Every translation unit is compiled by hipcc for gfx950 only, in parallel, then
linked into one shared library.  Packed-FP32 instructions are switched off
(``-packed-fp32-ops``) for every device compilation.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpa.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["status.cpp", "allocator.cpp", "prefix.cpp", "buddy.cpp", "api.cpp", "cache_write.hip", "decode.hip",
           "prefill.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-I/opt/rocm/include", "-Wall",
          "-Wno-unused-function"]
# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs (gfx950 allows
# it); otherwise the compiler parks them in AGPRs and copies them back and
# forth around every softmax step of the prefill kernel.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++", "-D__HIP_PLATFORM_AMD__", *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    return obj, errs


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, errs in results:
        if errs and verbose:
            print(errs, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
