"""Build libsa.so (the HIP kernels and the C-ABI entry points) for gfx950, in-tree.

Usage: python -m sparse_latent_attention_attn_amd.build_lib  (or call build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsa.so")
SOURCES = ["sa_api.cpp", "attn_fwd.hip", "aux_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed f32 vector instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with AGPR accumulators the compiler copies all of O to
    # VGPRs on every key tile for the (rarely taken) softmax rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(extra_flags: list[str] | None = None, out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
