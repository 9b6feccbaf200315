"""Build the CPU oracle (test infrastructure) with gcc.

``python -m oracle.build`` or ``oracle.build.build()`` compiles
``kvc_oracle.c`` into ``liboracle.so`` next to this file.  ``mutant`` builds a
copy with a planted mistake (``-DKVCO_MUTANT=n``) into ``out_dir``; only the
mutation tests use that.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvc_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(out: str = LIB, mutant: int = 0, verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-Werror", SRC, "-o", out + ".tmp", "-lm"]
    if mutant:  # a planted mistake may leave a variable unused
        cmd.remove("-Werror")
        cmd.insert(1, f"-DKVCO_MUTANT={int(mutant)}")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
