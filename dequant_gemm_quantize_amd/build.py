"""Build libw4.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m dequant_gemm_quantize_amd.build        # or __graft_entry__.build()

The library lands next to this file as ``libw4.so``; the Python binding loads
it from there.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libw4.so")
# measurement kernels (streaming read, matrix-instruction loops) for the
# roofline denominators; a library of their own, outside the method's ABI
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB_PATH = os.path.join(HERE, "libw4peaks.so")

SOURCES = ["api.cpp", "quant.hip", "gemv_generic.hip", "gemv_dot2.hip", "gemv_mfma.hip", "gemv_quad.hip", "gemv_decode.hip", "gemm_mfma.hip", "gemm_w4a8.hip", "gemv_w4a8.hip", "gemv_w4a8_mfma.hip", "gptq.hip"]

ARCH = os.environ.get("W4_OFFLOAD_ARCH", "gfx950")

# Flags that matter for bit-exactness and for the hardware:
#  * correctly rounded fp32 divide (the quantizer divides by the scale), and
#    denormals kept (fp16-subnormal scales are legal), no fast-math;
#  * packed-fp32 VALU instructions disabled (plain float code only);
#  * one code object for gfx950, no other targets.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}")
    if verbose and res.stdout.strip():
        print(res.stdout, flush=True)
    return res.stdout


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libw4.so (and libw4peaks.so); returns
    libw4.so's path."""
    _build_lib(SOURCES, LIB_PATH, verbose, jobs)
    _build_lib(PEAKS_SOURCES, PEAKS_LIB_PATH, verbose, jobs)
    return LIB_PATH


def _build_lib(sources, lib_path: str, verbose: bool, jobs: int) -> None:
    cc = hipcc()
    srcs = [s for s in sources if os.path.exists(os.path.join(CSRC, s))]
    with tempfile.TemporaryDirectory(prefix="w4build_") as tmp:
        objs = []
        procs = []
        for s in srcs:
            obj = os.path.join(tmp, s + ".o")
            lang = ["-x", "hip"] if s.endswith(".hip") else []
            cmd = [cc, *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, s), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        tmp_lib = os.path.join(tmp, os.path.basename(lib_path))
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        shutil.copyfile(tmp_lib, lib_path + ".tmp")
        os.replace(lib_path + ".tmp", lib_path)


def _wait(item, verbose):
    cmd, proc = item
    out, _ = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
