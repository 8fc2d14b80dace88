"""Compile the C oracle into oracle/liboracle.so (gcc, no intrinsics, no contraction)."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
