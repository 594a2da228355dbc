"""Build the HIP library libmxgemm.so in-tree for gfx950 (hipcc, no JIT).

Run ``python -m block_scaled_precision_e4m3_amd._build`` or call ``build()``.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
# One translation unit per group of kernel instantiations, compiled in parallel,
# then linked into one shared library (no relocatable device code: every unit
# carries its own kernels).
SOURCES = [os.path.join(CSRC, f) for f in ("mxgemm.hip", "launch_t256_bf16_f32.hip", "launch_t256_bf16_c16.hip",
                                           "launch_t128_bf16_f32.hip", "launch_t128_bf16_c16.hip",
                                           "launch_t256_proj.hip", "launch_fp8.hip", "launch_t256_mj.hip",
                                           "launch_t128_mj.hip", "probes.hip")]
LIB = os.path.join(PKG_DIR, "libmxgemm.so")
OBJ_DIR = os.path.join(PKG_DIR, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmxgemm.so")
    return exe


def build(verbose=False, extra_flags=(), jobs=None):
    """Compile libmxgemm.so (always recompiles every unit). Returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.basename(src).replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    errors = []
    for src, proc in zip(SOURCES, procs):
        out, _ = proc.communicate()
        if proc.returncode != 0:
            errors.append(f"{os.path.basename(src)}:\n{out}")
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
