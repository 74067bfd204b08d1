"""Compiles the CPU oracle (oracle.cpp) into liboracle.so with g++.

No -ffast-math and no FMA: the quantiser must round exactly as written
(x86-64 baseline code has no fused multiply-add).  `python oracle/build.py
--sanitize` builds _build/san/liboracle_san.so with AddressSanitizer and
UndefinedBehaviorSanitizer for a checking run of the CPU tests (loaded when
ORACLE_LIBRARY names it).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(HERE, "liboracle.so")


def build() -> str:
    src = os.path.join(HERE, "oracle.cpp")
    out = library_path()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sanitized() -> str:
    src = os.path.join(HERE, "oracle.cpp")
    sandir = os.path.join(os.path.dirname(HERE), "_build", "san")
    os.makedirs(sandir, exist_ok=True)
    out = os.path.join(sandir, "liboracle_san.so")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    import sys
    print(build_sanitized() if "--sanitize" in sys.argv[1:] else build())
