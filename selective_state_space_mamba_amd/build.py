"""Builds libmamba_scan.so (the gfx950 HIP kernels and their C ABI) in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmamba_scan.so")
SOURCES = [os.path.join(HERE, "csrc", "mamba_scan.hip")]
DEPS = SOURCES + [os.path.join(HERE, "csrc", f) for f in ("scan_kernels.h", "device_math.h")] + [
    os.path.join(ROOT, "include", "mamba_scan.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 instructions (v_pk_fma_f32 and friends) are switched off for the
# device code; hipcc's host pass warns that it does not know the feature.
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-shared", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(force: bool = True, extra_flags=(), out: str | None = None) -> str:
    """Compile the library.  With force=False, only when a source is newer."""
    out = out or LIB
    if not force and os.path.exists(out) and all(os.path.getmtime(out) >= os.path.getmtime(d) for d in DEPS):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra_flags) + ["-o", tmp] + SOURCES
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
