"""Compile the float64 CPU oracle (oracle/gdn_oracle.c, gdn_oracle_bwd.c, gdn_oracle_kda.c) into
oracle/libgdn_oracle.so with gcc.

Test infrastructure: the oracle is a checker, not part of the product path."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
SRC_BWD = os.path.join(HERE, "gdn_oracle_bwd.c")
SRC_KDA = os.path.join(HERE, "gdn_oracle_kda.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(x) for x in (SRC, SRC_BWD, SRC_KDA)):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           SRC, SRC_BWD, SRC_KDA, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
