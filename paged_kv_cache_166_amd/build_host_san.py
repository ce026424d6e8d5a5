"""Host-only build of the allocator, prefix index and buddy arena with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, no HIP code), for the
sanitizer run of the host tests (``tests/test_host_sanitizers.py``).

The library holds only the host C++ (``status.cpp``, ``allocator.cpp``,
``prefix.cpp``, ``buddy.cpp``); the binding loads it instead of libpa.so
when ``PA_HOST_LIB`` names it.  Python itself is not instrumented, so the
ASan runtime is preloaded into the interpreter that loads it.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(ROOT, "_build", "libpa_host_san.so")
SOURCES = ["status.cpp", "allocator.cpp", "prefix.cpp", "buddy.cpp"]
CXX = os.environ.get("CXX_HOST", "g++")


def build():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-shared", "-fPIC", "-Wall", "-Wno-unused-function",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-I/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__", *[os.path.join(CSRC, s) for s in SOURCES], "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed: {' '.join(cmd)}\n{r.stderr}")
    return OUT


def runtime_preload():
    """Path of the ASan runtime the sanitized library was linked against."""
    r = subprocess.run([CXX, "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build())
