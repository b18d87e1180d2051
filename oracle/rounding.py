"""Diagnostic oracle variant that rounds the way the bf16 kernels do
(oracle side; TEST INFRASTRUCTURE ONLY -- see the package docstring).

The float64 definition in oracle.attention is the parity target.  This
variant repeats it with the bf16 kernels' storage roundings applied at the
same points -- P rounded to bf16 before it weights V and dO, dS rounded to
bf16 before the dQ and dK products, outputs rounded once to bf16 -- so that
its distance from the float64 definition estimates the error floor that bf16
storage alone imposes.  It is reported beside the GPU error and is not a
gate.  Rounding uses PyTorch's CPU conversion, which takes a float64
value to float32 and then to bfloat16, each to nearest with ties to even:
the kernels round float32 values.  Pinned by tests/test_oracle_rounding.py
(an independent rounding written from the format, a scalar-loop twin that
must match bit for bit and fails with any one rounding left out, and a
hand-worked case).
"""

import numpy as np
import torch

from oracle import attention as A


def bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def forward_head(q, k, v, scale):
    p = A.probabilities(q, k, scale)
    o = bf16(p) @ np.asarray(v, dtype=np.float64)
    return bf16(o)


def backward_head(q, k, v, do, scale):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    sc = float(np.float32(scale))
    p = A.probabilities(q, k, scale)
    o = bf16(bf16(p) @ v)
    dv = bf16(bf16(p).T @ do)
    dp = do @ v.T
    row = (do * o).sum(axis=1, keepdims=True)   # the row term from the stored output
    ds = bf16(p * (dp - row))
    dq = bf16(sc * (ds @ k))
    dk = bf16(sc * (ds.T @ q))
    return dq, dk, dv
