"""Build libuaa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

``python -m sequence_attention_dits_amd.build`` or ``build_library()``.
Every source under csrc/ is compiled by hipcc for gfx950 only, in parallel,
then linked into ``sequence_attention_dits_amd/libuaa.so``.  Packed-fp32
instruction forms are disabled for all device code.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libuaa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "permute.hip", "merge.hip", "attn_fp32.hip", "attn_bf16.hip", "attn_p32.hip", "attn_bwd.hip", "attn_bwd_fp32.hip"]
HEADERS = ["internal.h", "attn_common.h"]

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function", "-Wno-inline-asm",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_id() -> str:
    """sha256 over every source and header the library is built from (and
    the build flags): built into the library, where uaa_build_id() returns
    it, and compared by the binding at load time, so a library left over
    from other sources is refused instead of run."""
    import hashlib
    h = hashlib.sha256()
    for name in SOURCES + HEADERS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(HERE, "..", "include", "uaa.h"), "rb") as f:
        h.update(b"uaa.h\0" + f.read())
    h.update(" ".join(CFLAGS).encode())
    return h.hexdigest()


def _compile(src: str, build_id: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, '-DUAA_BUILD_ID="%s"' % build_id, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build_library(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    build_id = source_id()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_id), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    # every kernel the library launches must be defined in it: an undefined
    # kernel symbol would only surface when the library is loaded
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [line for line in nm.stdout.splitlines() if "uaa" in line]
    if missing:
        os.remove(tmp)
        raise RuntimeError("libuaa.so has undefined symbols of its own:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
