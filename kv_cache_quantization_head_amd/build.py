"""Build the qkv HIP library (libqkv.so) in-tree for gfx950.

Usage: python -m kv_cache_quantization_head_amd.build [-v]
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqkv.so")
SOURCES = ["api.hip", "kernels.hip", "plan.cpp"]
ARCH = os.environ.get("QKV_OFFLOAD_ARCH", "gfx950")

# -ffp-contract=off: the codec's fp32 arithmetic is specified operation by
#   operation (fused multiply-adds are written explicitly as fmaf);
# -fno-gpu-flush-denormals-to-zero: IEEE subnormals in fp32;
# -packed-fp32-ops off: no packed fp32 VALU instructions are generated;
# -amdgpu-mfma-vgpr-form: MFMA accumulators stay in VGPRs (the k-means
#   screening reads every accumulator right after its MFMA).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the qkv library needs ROCm")
    return exe


def build(verbose=False):
    """Compile libqkv.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqkv.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
