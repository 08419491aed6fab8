"""Builds libmamba_scan.so (the gfx950 HIP kernels and their C ABI) in-tree.

The kernels are instantiated in eight translation units (the channel-block,
step and backward kernels, and the row kernels; each per element type x
input-term rule) compiled in parallel next to the host layer, then linked.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmamba_scan.so")
HOST = os.path.join(CSRC, "mamba_scan.hip")
INST = os.path.join(CSRC, "scan_inst.hip")
ROWS = os.path.join(CSRC, "row_inst.hip")
SOURCES = [HOST, INST, ROWS]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("scan_launch.h", "scan_kernels.h", "scan_row.h", "scan_bwd.h", "conv_kernels.h",
                                                  "device_math.h")] + [
    os.path.join(ROOT, "include", "mamba_scan.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# (bf16, exact) flags of the four instantiation units
VARIANTS = [(1, 0), (1, 1), (0, 0), (0, 1)]

# Packed FP32 instructions (v_pk_fma_f32 and friends) are switched off for the
# device code; hipcc's host pass warns that it does not know the feature.
# Floating-point contraction is off: every kernel rounds exactly as its source
# is written (fused multiply-adds only where __builtin_fmaf says so), so two
# kernels that compute the same value -- e.g. the pair form of the
# bidirectional scan and the per-direction rows plus merge -- agree bit for
# bit whatever the surrounding code lets the compiler fuse.
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), res.stdout))


def build(force: bool = True, extra_flags=(), out: str | None = None) -> str:
    """Compile the library.  With force=False, only when a source is newer."""
    out = out or LIB
    if not force and os.path.exists(out) and all(os.path.getmtime(out) >= os.path.getmtime(d) for d in DEPS):
        return out
    with tempfile.TemporaryDirectory(prefix="mscan_build_") as tmp:
        jobs = [[HIPCC] + FLAGS + list(extra_flags) + ["-c", "-o", os.path.join(tmp, "host.o"), HOST]]
        for unit in (INST, ROWS):
            for bf16, exact in VARIANTS:
                obj = os.path.join(tmp, "%s_%d%d.o" % (os.path.basename(unit).split(".")[0], bf16, exact))
                jobs.append([HIPCC] + FLAGS + list(extra_flags) +
                            ["-DMSCAN_INST_BF16=%d" % bf16, "-DMSCAN_INST_EXACT=%d" % exact, "-c", "-o", obj, unit])
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
            list(ex.map(_run, jobs))
        objs = [j[j.index("-o") + 1] for j in jobs]
        tmp_out = out + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_out] + objs)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
