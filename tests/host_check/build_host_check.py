"""Build tests/host_check/lla_host_check: the library's host code (every
source under csrc/, compiled host-only: no device code) plus the driver in
lla_host_check.cpp, with AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitizer flags apply to the host pass only (-Xarch_host), and the link
runs through clang++ directly.  Objects go to _build/host_check/ at the
repository root; the executable is rebuilt when any source is newer."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "looped_transformer_latent_amd", "csrc")
OBJ = os.path.join(ROOT, "_build", "host_check")
EXE = os.path.join(OBJ, "lla_host_check")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-g", "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _sources():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from looped_transformer_latent_amd import build
    return [os.path.join(CSRC, s) for s in build.LLA_SOURCES]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if os.path.exists(obj) and os.path.getmtime(obj) >= max(
            os.path.getmtime(src), *(os.path.getmtime(os.path.join(CSRC, h)) for h in
                                     ("lla_internal.h", "lla_device.h")),
            os.path.getmtime(os.path.join(ROOT, "include", "lla.h"))):
        return obj
    if src.endswith(".cpp"):
        cmd = [CLANGXX, *COMMON, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, "--offload-arch=gfx950", *COMMON, "-Xarch_device", "-O3", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", *SAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = _sources() + [os.path.join(HERE, "lla_host_check.cpp")]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = [CLANGXX, "-fsanitize=address,undefined", *objs, "-o", EXE, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return EXE


if __name__ == "__main__":
    print(build())
