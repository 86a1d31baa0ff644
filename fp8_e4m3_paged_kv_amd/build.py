"""Build libfp8kv.so (gfx950) in-tree with hipcc.

    python -m fp8_e4m3_paged_kv_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfp8kv.so")
# measurement kernels for the benchmark (HBM streams, launch floor)
PROBES_LIB = os.path.join(PKG, "libfp8kv_probes.so")
PROBES_SRC = os.path.join(PKG, "csrc", "probes", "hbm_probes.hip")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep packed fp32 (v_pk_*_f32) out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online-softmax rescale multiplies them
    # with VALU ops, which cannot read AGPRs without a copy per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    csrc = os.path.join(PKG, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) +
                  glob.glob(os.path.join(csrc, "*.cpp")))


def _hipcc(srcs, out, verbose):
    hipcc = os.environ.get("HIPCC", "hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"),
                                   "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Build libfp8kv.so and the benchmark's probe library."""
    _hipcc(sources(), LIB, verbose)
    _hipcc([PROBES_SRC], PROBES_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
