"""Builds libtria.so (the C-ABI library) in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instructions disabled (hipcc still
vectorises ordinary float code otherwise) and with the default IEEE-correct fp32
division that the quantiser's bit-exact contract relies on.

`python block_sparse_mixed_head_amd/build.py --sanitize` builds a checking variant,
_build/san/libtria_san.so, for the CPU tests only: the host code (capi.cpp: argument
validation, schedule and page-table builders, the allocator) compiled by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer, linked with the unchanged GPU
objects.  The binding loads it when TRIA_LIBRARY names it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["capi.cpp", "quantize.hip", "prefill.hip", "pack.hip", "decode.hip", "peaks.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


# peaks.hip: the MFMA issue loops keep their accumulators in VGPRs; in the AGPR form
# the register allocator rotates the loop-carried tuples through accvgpr moves, which
# would understate the ceiling the loops are there to measure.
EXTRA_FLAGS = {"peaks.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def library_path() -> str:
    return os.path.join(HERE, "libtria.so")


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ["hipcc", *FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build_sanitized() -> str:
    """Host code with ASan + UBSan (g++), GPU objects as in build(); see the module doc."""
    objdir = os.path.join(ROOT, "_build")
    sandir = os.path.join(objdir, "san")
    os.makedirs(sandir, exist_ok=True)
    gpu = [s for s in SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=len(gpu)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), gpu))
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    capi = os.path.join(sandir, "capi.o")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", INCLUDE, "-I", CSRC, *san, "-c", os.path.join(CSRC, "capi.cpp"), "-o", capi]
    subprocess.run(cmd, check=True)
    out = os.path.join(sandir, "libtria_san.so")
    cmd = ["g++", "-shared", *san, capi, *objs, "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    subprocess.run(cmd, check=True)
    return out


def build() -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_sanitized() if "--sanitize" in sys.argv[1:] else build())
