"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain gcc, -O2, no fused multiply-add contraction and no fast-math, so the
binary64 arithmetic is exactly what oracle.c spells out.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Werror"]


def build(sanitize: bool = False, out: str = None, src: str = None, werror: bool = True) -> str:
    """Compile oracle.c (or another source file); returns the library path."""
    out = out or (LIB if not sanitize else os.path.join(HERE, "liboracle_san.so"))
    src = src or SRC
    flags = [f for f in CFLAGS if werror or f != "-Werror"]
    if sanitize:
        flags += ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    tmp = out + ".tmp"
    subprocess.run(["gcc", *flags, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
