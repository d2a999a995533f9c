"""Compile the CPU oracle and its brute-force checker into liboracle.so.

Test infrastructure only (see moe_oracle.h)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["moe_oracle.cpp", "brute.cpp"]


def build(verbose: bool = False, out: str = None, sources_dir: str = None) -> str:
    sdir = sources_dir or HERE
    out = out or os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
           "-I", HERE] + [os.path.join(sdir, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
