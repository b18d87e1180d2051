"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws random numbers,
applies the input projection that produces per-head queries, keys and values
from token activations, splits heads, and rounds to the storage dtype.  Both
the GPU tests/bench and the CPU oracle consume the tensors it returns.

Shapes stand in for the model sizes the pages train (no dataset or trained
weights are used; activations are Gaussian):

* ``tiny_fp32``       1 x 4 heads x 64 tokens x 16, float32, iid N(0, 1)
* ``char_gpt``        64 x 6 x 256 x 64  -- the nanoGPT README's Shakespeare
                      character model (6 layers, 6 heads, 384 dims, 256 ctx)
* ``gpt2_124m``       12 x 12 x 1024 x 64 -- GPT-2 124M (768 dims, 12 heads)
* ``gpt2_xl``         4 x 25 x 1024 x 64  -- GPT-2 with 48 layers and
                      d_model 1600 (minGPT README notes), head size 64
* ``gpt3_2048``       1 x 96 x 2048 x 128 -- GPT-3 style layer that always
                      uses the full 2048 context (minGPT README notes)

Recipe ``projection`` (all bf16 workloads), drawn from
``numpy.random.default_rng(seed)`` in this order: x ~ N(0, 1) of shape
``[B, T, C]`` with C = H * D; W_q, W_k, W_v ~ N(0, 0.02) (standard deviation
0.02, the minGPT README's weight init), each ``[C, C]``; dO ~ N(0, 0.01) of
shape ``[B, H, T, D]``.  q = x W_q (float32 product on the CPU), reshaped to
``[B, T, H, D]`` and transposed to ``[B, H, T, D]``; likewise k and v.  Every
tensor is then rounded once, round-to-nearest-even, to bfloat16.

Recipe ``iid`` (the float32 workload): q, k, v, dO ~ N(0, 1), drawn directly
in ``[B, H, T, D]`` in that order.

The softmax scale is 1/sqrt(D) rounded to float32.
"""

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str  # "bf16" or "f32"
    recipe: str  # "projection" or "iid"
    what: str

    @property
    def N(self):
        return self.B * self.H


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32", 1, 4, 64, 16, "f32", "iid",
                 "tiny causal attention, float32"),
        Workload("char_gpt", 64, 6, 256, 64, "bf16", "projection",
                 "character-level GPT attention layer (n_embd 384, ctx 256)"),
        Workload("gpt2_124m", 12, 12, 1024, 64, "bf16", "projection",
                 "GPT-2 124M attention layer (n_embd 768, ctx 1024)"),
        Workload("gpt2_xl", 4, 25, 1024, 64, "bf16", "projection",
                 "GPT-2 48-layer d_model 1600 attention layer (ctx 1024)"),
        Workload("gpt3_2048", 1, 96, 2048, 128, "bf16", "projection",
                 "GPT-3 style layer, d_model 12288, full 2048 context"),
    )
}


def default_scale(D):
    """1/sqrt(D) rounded to float32 (returned as a Python float)."""
    return float(np.float32(1.0 / np.sqrt(D)))


def _to_storage(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(B, H, T, D, dtype="bf16", seed=0, recipe="projection"):
    """Draw one seeded set of attention inputs.

    Returns a dict with CPU torch tensors ``q, k, v, do`` of shape
    ``[B, H, T, D]`` in the storage dtype (bfloat16 or float32) and the
    float32-exact ``scale``.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.default_rng(seed)
    shape = (B, H, T, D)
    if recipe == "iid":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        do = rng.standard_normal(shape, dtype=np.float32)
        out = {n: _to_storage(a, dtype) for n, a in
               (("q", q), ("k", k), ("v", v), ("do", do))}
    elif recipe == "projection":
        C = H * D
        x = torch.from_numpy(rng.standard_normal((B * T, C), dtype=np.float32))
        out = {}
        for n in ("q", "k", "v"):
            w = rng.standard_normal((C, C), dtype=np.float32)
            w *= np.float32(0.02)
            y = torch.matmul(x, torch.from_numpy(w))  # [B*T, C] float32
            del w
            y = y.view(B, T, H, D).permute(0, 2, 1, 3).contiguous()
            out[n] = y.to(torch.bfloat16) if dtype == "bf16" else y
            del y
        do = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01)
        out["do"] = _to_storage(do, dtype)
    else:
        raise ValueError("unknown recipe " + repr(recipe))
    out["scale"] = default_scale(D)
    return out


def workload_inputs(name, seed=0):
    """Inputs for one named workload (see the module docstring)."""
    w = WORKLOADS[name]
    return make_inputs(w.B, w.H, w.T, w.D, w.dtype, seed, w.recipe)

