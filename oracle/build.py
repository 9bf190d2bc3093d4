"""Compile the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain C11 with OpenMP, -O2, no fast-math and no FMA contraction, so every
double-precision product and sum happens in the order the source states.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    src = os.path.join(HERE, "oracle.c")
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(src):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


SANITIZED = os.path.join(HERE, "oracle_sanitized")


def build_sanitized(selfcheck: bool = False) -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer linked
    into sanitize_main.c, a driver of every entry point on tiny shapes (a
    host-only executable; any sanitizer report ends it with a failure).
    selfcheck builds the driver's planted out-of-bounds read instead, to show
    that the build is instrumented."""
    out = SANITIZED + ("_selfcheck" if selfcheck else "")
    tmp = out + ".tmp"
    cmd = ["gcc", *(["-DSANITIZER_SELFCHECK"] if selfcheck else []), "-std=gnu11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", tmp,
           os.path.join(HERE, "oracle.c"), os.path.join(HERE, "sanitize_main.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
