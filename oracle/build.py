"""Compiles the CPU oracle (oracle.cpp) into liboracle.so with g++.

No -ffast-math and no FMA: the quantiser must round exactly as written
(x86-64 baseline code has no fused multiply-add).
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


if __name__ == "__main__":
    print(build())
