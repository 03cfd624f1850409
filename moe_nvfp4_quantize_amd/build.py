"""Build libnvfp4.so in-tree with hipcc for gfx950.

    python -m moe_nvfp4_quantize_amd.build        # or: from ... import build; build.build()

Every source is compiled to an object under ``_build/`` next to this file and
linked into ``libnvfp4.so`` beside it; the benchmark's HBM ceiling kernels
(``csrc/ceiling.hip``, not part of the layer) go into ``libnvfp4_ceiling.so``.
The device code is built with:
  * ``-ffp-contract=off``: the quantizer's float32 steps are specified one
    rounding at a time; no multiply-add fusion may merge them;
  * ``-fhip-fp32-correctly-rounded-divide-sqrt``: its two divisions per block
    are IEEE correctly rounded;
  * packed-FP32 instructions disabled (``-packed-fp32-ops``).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "fp8_gemm.hip", "moe.hip"]
CEILING_SOURCES = ["ceiling.hip"]
LIB_CEILING = os.path.join(HERE, "libnvfp4_ceiling.so")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libnvfp4.so")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, warn


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile every source and link libnvfp4.so (and libnvfp4_ceiling.so);
    returns the path of libnvfp4.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for obj, warn in results.values():
        if warn.strip() and verbose:
            print(warn, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in CEILING_SOURCES], LIB_CEILING)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
