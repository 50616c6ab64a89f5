"""Build libsketchssm.so (HIP kernels for gfx950 + the C ABI) in-tree."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsketchssm.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 ops are disabled for all device code.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
SOURCES = ["sk_api.cpp", "sk_m2.hip", "sk_gdn.hip", "sk_kda.hip", "sk_m2_f32.hip", "sk_gdn_f32.hip",
           "sk_kda_f32.hip", "sk_noalloc.hip"]


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + CFLAGS + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _stale(src: str, tag: str) -> bool:
    """An object is stale when it is missing or older than its source or any
    header it may include (the csrc headers and include/sketchssm.h)."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src), os.path.join(ROOT, "include", "sketchssm.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".inc"))]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(jobs: int = 8, extra=(), out: str = LIB, incremental: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library.
    extra: additional compiler flags (e.g. -D tuning macros); out: library path;
    incremental: recompile only the objects older than their sources."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if out == LIB else "_" + os.path.basename(out).replace(".so", "")

    def obj_of(src):
        if incremental and not extra and not _stale(src, tag):
            return os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
        return _compile(src, extra, tag)

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(obj_of, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(incremental="--incremental" in sys.argv))
    sys.exit(0)
