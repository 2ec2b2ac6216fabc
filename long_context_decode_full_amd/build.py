"""Builds libhs2.so (HIP kernels for gfx950 + the C-ABI host layer) in-tree with hipcc.

Each source compiles to its own object in parallel, then hipcc links the shared
library.  The library embeds a hash of every source and header it is built from
(hs2_build_id), so a stale binary is detectable."""
import hashlib
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhs2.so")
SOURCES = ["hs2_scan.hip", "hs2_scan_mfma.hip", "hs2_chunk_mfma.hip", "hs2_select.hip", "hs2_select_fast.hip",
           "hs2_bridge.hip", "hs2_swa.hip", "hs2_scratch.hip", "hs2_api.cpp"]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libhs2.so)")


def source_files():
    """Every file the library is built from: the kernel and host sources, the internal
    headers and the public header, in a fixed order."""
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".cpp", ".h")))
    return files + [os.path.join(INCLUDE, "hs2.h")]


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 over the sources' names and contents."""
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _common_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden",
        # packed fp32 VALU forms stay disabled on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        f"-DHS2_BUILD_ID=\"{source_hash()}\"",
    ]


def command(out=LIB):
    """One hipcc invocation that compiles and links everything (reference form)."""
    return [hipcc(), *_common_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stderr


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    flags = _common_flags()
    with tempfile.TemporaryDirectory(prefix="hs2_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[cc, *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
            logs = list(ex.map(_run, cmds))
        tmp = LIB + ".tmp"
        logs.append(_run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    if verbose:
        print("".join(logs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
