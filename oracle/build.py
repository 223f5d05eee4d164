"""Build oracle/liboracle.so from cd_oracle.c with gcc.

Test infrastructure: the library is loaded only by tests/, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no FMA contraction: each fp32/fp64 operation in the source
# is the IEEE operation that executes.
CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-math-errno", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle; returns the library path."""
    out = LIB if not sanitize else os.path.join(HERE, "liboracle_san.so")
    if not force and os.path.exists(out) and \
            os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    flags = list(CFLAGS)
    if sanitize:
        flags += ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *flags, "-o", tmp, SRC, "-lm"])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
