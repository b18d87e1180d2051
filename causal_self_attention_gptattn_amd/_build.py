"""Build libgptattn.so in-tree with hipcc for gfx950.

Usage: ``python -m causal_self_attention_gptattn_amd._build [--resource-usage]``
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgptattn.so")
SOURCES = ["gptattn_api.hip", "attn_bf16.hip", "attn_d64.hip", "attn_d128.hip", "attn_decode.hip",
           "attn_f32.hip"]
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose=False, resource_usage=False):
    """Compile every HIP source into ``libgptattn.so``; raises on failure."""
    cmd = [hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    os.replace(LIB + ".tmp", LIB)
    if verbose and out.strip():
        print(out)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
