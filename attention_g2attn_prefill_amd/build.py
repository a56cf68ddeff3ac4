"""Build libg2attn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into attention_g2attn_prefill_amd/libg2attn.so.  The sha256 of the sources
(csrc/, the public header, the flags) is baked into the library and returned
by g2attn_build_id(), so a run can tell whether the binary it loaded was built
from the sources beside it.
"""
import hashlib
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libg2attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function",
                "-I", os.path.join(ROOT, "include"), "-I", CSRC]


HEADER = os.path.join(ROOT, "include", "g2attn.h")
BUILD_ID_TAG = b"g2attn-build-id:"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def source_hash() -> str:
    """sha256 of everything the library is built from: every file under csrc/
    (name and bytes), the public header and the compiler flags."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, name)
        if os.path.isfile(path):
            h.update(name.encode())
            with open(path, "rb") as fh:
                h.update(fh.read())
    with open(HEADER, "rb") as fh:
        h.update(b"g2attn.h")
        h.update(fh.read())
    h.update(" ".join(DEVICE_FLAGS).replace(ROOT, "").encode())
    return h.hexdigest()


def built_id(lib_path: str = LIB):
    """The source hash baked into a built library (read from its bytes, without
    loading it), or None if there is no library or no id in it."""
    try:
        with open(lib_path, "rb") as fh:
            data = fh.read()
    except OSError:
        return None
    m = re.search(re.escape(BUILD_ID_TAG) + rb"([0-9a-f]{64})", data)
    return m.group(1).decode() if m else None


def is_current() -> bool:
    return built_id() == source_hash()


def _compile(src: str, verbose: bool, build_id: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, f'-DG2ATTN_BUILD_ID="{build_id}"', "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    build_id = source_hash()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_id), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
