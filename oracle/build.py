"""Compile the CPU fp64 oracle (test infrastructure) into oracle/libg2oracle.so.

Plain C99 + OpenMP with gcc; nothing from the HIP library is compiled in.  The
sha256 of the source and the flags is baked into the library's bytes, so the
tests can tell a stale build from a current one without loading it.
"""
import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "g2_oracle.c")
LIB = os.path.join(HERE, "libg2oracle.so")
FLAGS = ["-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC"]
ID_TAG = b"g2oracle-build-id:"


def source_hash() -> str:
    h = hashlib.sha256()
    with open(SRC, "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def built_id():
    try:
        with open(LIB, "rb") as fh:
            data = fh.read()
    except OSError:
        return None
    m = re.search(re.escape(ID_TAG) + rb"([0-9a-f]{64})", data)
    return m.group(1).decode() if m else None


def is_current() -> bool:
    return built_id() == source_hash()


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *FLAGS, f'-DG2O_BUILD_ID="{source_hash()}"', "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
