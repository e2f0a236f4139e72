"""Build libdllm_cache.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m diffusion_kv_cache_amd.build  (or build() from Python).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdllm_cache.so")
SOURCES = ["api.hip", "refresh.hip", "refresh_splitk.hip", "attention.hip", "attention_fwd.hip",
           "attention_fused.hip", "attention_facache.hip", "drift.hip", "schedule.hip", "fp8_linear.hip", "unfused.hip"]
ARCH = os.environ.get("DLLM_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU ops off (no v_pk_* fp32 instructions in any kernel)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-source additions.  The attention kernels keep their MFMA accumulators in ordinary
# VGPRs: with accumulation registers the compiler copied all 64 output accumulators out and
# back on every key tile (the lazily rescaled softmax state is loop-carried through a branch),
# and the mass pass read every score out of them with one extra instruction each.
# NaNs are not honoured there either (no canonicalising max before every fmaxf of a score):
# scores of finite inputs are finite, and masked keys are -inf, which stays honoured.
EXTRA = {"attention_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attention_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attention_facache.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "fp8_linear.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = ["hipcc", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if out.strip():
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.check_call(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
