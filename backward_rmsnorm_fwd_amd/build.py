"""Build the HIP library ``librmsnorm.so`` in-tree with hipcc for gfx950.

Usage: ``python -m backward_rmsnorm_fwd_amd.build [--resource-usage]``.
``--resource-usage`` also prints each kernel's VGPR/SGPR/LDS/spill figures
(compiler remark ``kernel-resource-usage``) of the compiled kernels.
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
# Translation units: (source, extra hipcc arguments, object name).  The
# full-width kernel instantiations compile once per dtype from one source.
UNITS = [(os.path.join(CSRC, "rmsnorm_api.hip"), [], "rmsnorm_api.o")]
UNITS += [(os.path.join(CSRC, "rmsnorm_fast_inst.hip"), [f"-DRMSNORM_INST_DT={dt}"],
           f"rmsnorm_fast_inst_{dt}.o") for dt in ("kF32", "kF16", "kBF16")]
UNITS += [(os.path.join(CSRC, f), [], f.replace(".hip", ".o")) for f in (
    "rmsnorm_split.hip", "layernorm.hip", "layernorm_rows.hip", "layernorm_split.hip",
    "fused_add.hip",
    "fused_cast.hip")]
SOURCES = sorted({src for src, _, _ in UNITS})
LIB = os.path.join(HERE, "librmsnorm.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # IEEE-correct float32 division and square root in device code.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # Keep the compiler from forming packed-float32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose=False, resource_usage=False, jobs=None):
    """Compile the library (always; never skipped when one already exists).

    Each translation unit compiles in its own hipcc process (in parallel);
    the objects are then linked into one shared library."""
    jobs = jobs or min(len(UNITS), max(1, os.cpu_count() or 1))
    inc = ["-I", os.path.join(ROOT, "include")]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    with tempfile.TemporaryDirectory(prefix="rmsnorm_build_") as tmp:
        objs = [os.path.join(tmp, name) for _, _, name in UNITS]
        cmds = [[hipcc(), *FLAGS, *extra, *inc, *defs, "-c", src, "-o", obj]
                for (src, defs, _), obj in zip(UNITS, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        logs = []
        for cmd, (rc, out) in zip(cmds, results):
            logs.append(out)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{out}")
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                "-o", LIB + ".tmp"]
        rc, out = _run(link, verbose)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(LIB + ".tmp", LIB)
    if resource_usage or verbose:
        print("\n".join(logs))
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
