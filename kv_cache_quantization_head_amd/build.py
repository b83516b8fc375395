"""Build the qkv HIP library (libqkv.so) in-tree for gfx950.

Every source is compiled to an object in parallel, then the objects are
linked into libqkv.so.

Usage: python -m kv_cache_quantization_head_amd.build [-v]
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqkv.so")
SELFCHECK = os.path.join(HERE, "selfcheck_mfma_f64")
ARCH = os.environ.get("QKV_OFFLOAD_ARCH", "gfx950")

# -ffp-contract=off: the codec's fp32 arithmetic is specified operation by
#   operation (fused multiply-adds are written explicitly as fmaf);
# -fno-gpu-flush-denormals-to-zero: IEEE subnormals in fp32;
# -packed-fp32-ops off: no packed fp32 VALU instructions are generated.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# per source: extra flags.  -amdgpu-mfma-vgpr-form keeps MFMA accumulators in
# VGPRs (the k-means screening reads every accumulator right after its MFMA).
SOURCES = {
    "api.hip": [],
    "encode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode.hip": [],
    "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "xlayer.hip": [],
    "plan.cpp": [],
}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the qkv library needs ROCm")
    return exe


def build(verbose=False):
    """Compile libqkv.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(OBJ, src + ".o")
        objs.append(obj)
        cmd = [hipcc()] + COMMON + extra + ["-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libqkv.so")
    os.replace(tmp, LIB)
    # the self-check of the fp64 matrix instruction's summation order (run by
    # the GPU tests; the cross-layer kernels rely on it)
    cmd = [hipcc()] + COMMON + ["-o", SELFCHECK, os.path.join(CSRC, "selfcheck_mfma_f64.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building selfcheck_mfma_f64")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
