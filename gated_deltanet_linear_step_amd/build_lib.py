"""Build libgdn.so (all HIP kernels + the C ABI) for gfx950, in-tree.

    python -m gated_deltanet_linear_step_amd.build_lib

hipcc cross-compiles for gfx950 without a GPU. Packed-FP32 instructions are
disabled for the device code (``-packed-fp32-ops``).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_conv.hip", "gdn_decode.hip", "gdn_prefill.hip",
           "gdn_prefill_generic.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # keep MFMA accumulators in ordinary VGPRs: the prefill carry scales
           # and converts its accumulators with VALU work every chunk
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           ] + [f"-D{d}" for d in defines] + ["-x", "hip"] + srcs + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx950 packed-fp32 feature; drop that notice
    for line in (res.stdout + res.stderr).splitlines():
        if "packed-fp32-ops" not in line and "unused during compilation" not in line:
            print(line, file=sys.stderr)
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
