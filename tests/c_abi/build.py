"""Compile the plain-C consumer of the C ABI (tests/c_abi/c_abi_check.c).

It links the HIP library (attention_g2attn_prefill_amd/libg2attn.so), the CPU
oracle (oracle/libg2oracle.so, test infrastructure) and the HIP runtime, with
gcc and no HIP device code, and finds both libraries next to the tree at run
time through its rpath.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "c_abi_check.c")
EXE = os.path.join(HERE, "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-o", EXE + ".tmp", SRC,
           "-L", os.path.join(ROOT, "attention_g2attn_prefill_amd"), "-lg2attn",
           "-L", os.path.join(ROOT, "oracle"), "-lg2oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../attention_g2attn_prefill_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
