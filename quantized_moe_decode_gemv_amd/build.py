"""Compile the gfx950 HIP library ``libqmoe.so`` in-tree with hipcc.

``build(timeline=True)`` (``python -m quantized_moe_decode_gemv_amd.build
--timeline``) compiles the profiling variant ``libqmoe_timeline.so`` instead:
the same sources with -DQMOE_TIMELINE, whose decode kernels write
s_memrealtime stamps (csrc/moe_timeline.h) that ``bench.py --timeline`` reads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmoe.so")
LIB_TIMELINE = os.path.join(HERE, "libqmoe_timeline.so")
SOURCES = ["moe_gemv.hip", "moe_egemv.hip", "moe_grouped.hip", "moe_api.cpp", "moe_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of generated code on purpose.
# MFMA results go to ordinary VGPRs (gfx950 allows either register file):
# in the AGPR form each 16x16 result of the tile kernels came back through
# four v_accvgpr_read before its fp32 sub-block affine, 10-18 % of their
# VALU instructions; outputs are bit-identical either way.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def build(verbose=False, timeline=False):
    """Always recompiles (the caller asked for a build)."""
    out = LIB_TIMELINE if timeline else LIB
    srcs = []
    for s in sources():
        if s.endswith(".cpp"):
            srcs += ["-x", "hip", s]
        else:
            srcs.append(s)
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + (["-DQMOE_TIMELINE"] if timeline else []) + srcs + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
