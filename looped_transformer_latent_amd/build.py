"""Build the HIP libraries in-tree for gfx950 with hipcc.

* ``liblla.so``      -- the LLA kernels and the C ABI of ``include/lla.h``.
* ``liblla_gen.so``  -- the device side of the seeded input generator.

Objects go to ``_build/`` at the repository root; the shared libraries are
written next to this file so that they travel with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

LLA_SOURCES = ["lla_api.hip", "lla_absorbed.hip", "lla_decode.hip", "lla_decode_g.hip", "lla_decode2d.hip", "lla_encode.hip", "lla_full.hip", "lla_merge.hip", "lla_prefill.hip", "lla_rope.hip"]
GEN_SOURCES = ["gen/lla_gen.hip"]

# Packed-fp32 VALU ops are disabled for every HIP source; hipcc's host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]

# Sources whose kernels issue global -> LDS copies from inline assembly that
# sets M0 itself (copy16_to_lds in lla_encode.hip): the build checks that the
# compiler keeps nothing else in M0 there.
M0_CHECKED = ["lla_encode.hip"]

LIB = os.path.join(PKG, "liblla.so")
GEN_LIB = os.path.join(PKG, "liblla_gen.so")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.replace("/", "_") + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def check_m0(src: str) -> None:
    """Device assembly of src: every M0 write must be the one directly before
    a global_load_lds_dwordx4, and no other instruction may name M0."""
    asm = os.path.join(OBJ, src.replace("/", "_") + ".s")
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    bad = m0_misuse(open(asm).read())
    if bad is not None:
        raise RuntimeError(f"{src}: M0 used outside the LDS copy blocks: {bad!r}")


def m0_misuse(text: str):
    """The first instruction of an assembly listing that names M0 other than
    an `s_mov_b32 m0, ...` directly followed by global_load_lds_dwordx4, or None."""
    lines = [ln.split(";")[0].strip() for ln in text.splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]
    for i, ln in enumerate(lines):
        ops = ln.replace(",", " ").split()
        if "m0" not in ops[1:]:
            continue
        if not (ops[0] == "s_mov_b32" and ops[1] == "m0" and i + 1 < len(lines)
                and lines[i + 1].startswith("global_load_lds_dwordx4")):
            return ln
    return None


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {out}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> list[str]:
    """Compile every HIP source (always: this is the does-it-build check)."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        lla_objs = list(ex.map(_compile, LLA_SOURCES))
        gen_objs = list(ex.map(_compile, GEN_SOURCES))
        list(ex.map(check_m0, M0_CHECKED))
    _link(lla_objs, LIB)
    _link(gen_objs, GEN_LIB)
    return [LIB, GEN_LIB]


if __name__ == "__main__":
    for p in build():
        print(p)
