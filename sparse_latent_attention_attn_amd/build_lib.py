"""Build libsa.so (the HIP kernels and the C-ABI entry points) for gfx950, in-tree.

Usage: python -m sparse_latent_attention_attn_amd.build_lib  (or call build()).

Each source is compiled to an object of its own (the translation units need different
accumulator settings, below), then the objects are linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed f32 vector instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA accumulators in VGPRs: the key loops with up to 128 accumulators per lane schedule
# best this way. The wide key loop (256 accumulators per lane) needs them in AGPRs.
VGPR_ACC = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = {
    "sa_api.cpp": [],
    "attn_fwd.hip": VGPR_ACC,
    "attn_fwd_wide.hip": [],
    "aux_kernels.hip": VGPR_ACC,
    "noalloc.hip": [],
    "indexer.hip": VGPR_ACC,
    "wo_proj.hip": [],
}

_NOISE = ("is not a recognized feature for this target", "(ignoring feature)")


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in _NOISE))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(extra_flags: list[str] | None = None, out: str = LIB) -> str:
    with tempfile.TemporaryDirectory(prefix="sa_build_") as tmpdir:
        objs = []
        for src, flags in SOURCES.items():
            obj = os.path.join(tmpdir, src + ".o")
            _run([HIPCC, *COMMON, *flags, *(extra_flags or []), "-c", "-o", obj, os.path.join(CSRC, src)])
            objs.append(obj)
        tmp = out + ".tmp"
        _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
