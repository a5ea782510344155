"""Build the HIP library ``libskiparse_amd.so`` in-tree for gfx950.

    python -m skiparse_sparse_attention_amd.build

Runs hipcc on the sources under ``csrc/``; cross-compiles without a GPU.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libskiparse_amd.so")
SOURCES = ["skiparse_api.cpp", "rope_remap.hip", "attn_fwd.hip", "attn_bwd.hip", "quant8.hip", "attn8_fwd.hip",
           "attn_rot.hip", "probes.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed-FP32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source into LIB; raise CalledProcessError on failure."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the GPU-only feature above
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise subprocess.CalledProcessError(res.returncode, cmd, output=msgs)
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    try:
        print(build(verbose=True))
    except subprocess.CalledProcessError as e:
        print(e.output, file=sys.stderr)
        sys.exit(1)
