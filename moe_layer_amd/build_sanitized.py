"""Build the library with AddressSanitizer and UndefinedBehaviorSanitizer on
its HOST code (argument checks, workspace sizing, launch set-up, the switch
policy), for CPU-side testing only:

    python -m moe_layer_amd.build_sanitized      # -> _build/san/libmoe_layer_amd.so

Device code is compiled as usual (no GPU sanitizer): on every hipcc line each
sanitizer flag is preceded by -Xarch_host.  The host-only .cpp sources go
through clang++ from the same toolchain, so that one sanitizer runtime (clang's,
loaded with LD_PRELOAD, see ASAN_RUNTIME) serves the whole library.  The tests
that use it (tests/test_sanitized_host.py) call only host paths: every call
fails its argument checks before anything is enqueued, or is host-only.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from . import build as B

OUT_DIR = os.path.join(B.ROOT, "_build", "san")
LIB = os.path.join(OUT_DIR, "libmoe_layer_amd.so")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
CXX_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return found[-1]


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", f"-I{B.INCLUDE}", f"-I{B.CSRC}", "-I/opt/rocm/include",
               "-D__HIP_PLATFORM_AMD__", *CXX_SAN, "-c", src, "-o", obj]
    else:
        cmd = [B.HIPCC, *[f for f in B.CFLAGS if f != "-O3"], "-O1", "-g", *HOST_SAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed on {src}:\n{r.stderr}")
    return obj


def build():
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(8) as pool:
        objs = list(pool.map(_compile, B.sources()))
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *HOST_SAN, "-o", LIB, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
