"""Builds libwfattn.so for gfx950 with hipcc (sources in csrc/, header in include/)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwfattn.so")
SOURCES = ["capi.hip", "dense.hip", "vsa.hip", "rope.hip", "noalloc.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU instructions.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def _record_revision() -> None:
    """Write the source revision next to the library, for runs on copies of the tree that carry
    no .git (the benchmark reports it)."""
    import json
    info = {"git": "unknown", "dirty": False}
    try:
        rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True, timeout=10)
        if rev.returncode == 0 and rev.stdout.strip():
            info["git"] = rev.stdout.strip()
            st = subprocess.run(["git", "status", "--porcelain", "--untracked-files=no", "--",
                                 os.path.relpath(CSRC, ROOT), os.path.relpath(INCLUDE, ROOT)],
                                cwd=ROOT, capture_output=True, text=True, timeout=10)
            info["dirty"] = bool(st.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(PKG, "build_info.json"), "w") as f:
        json.dump(info, f)
        f.write("\n")


def build(extra: list | None = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    extra = list(extra or [])
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    _record_revision()
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
