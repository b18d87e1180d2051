"""CPU check of gpu_helpers.rounding_bound: the first-order bound on what the
bf16 path's storage roundings can move each output by must contain the
deviation of a float64 computation that applies exactly those roundings
(weights before P V and P^T dO, the stored O that the row term is formed
from, dS before dS K and dS^T Q, every output once) from the float64
definition, element by element, with dropout, bands and offsets."""

import numpy as np
import pytest
import torch

from causal_self_attention_gptattn_amd import workloads as W
from gpu_helpers import rounding_bound
from oracle import attention as A, philox


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def rounded_head(q, k, v, do, scale, off, win, keep, p):
    """Forward and backward of one head with the bf16 kernels' storage roundings."""
    sc = float(np.float32(scale))
    w = A.probabilities(q, k, scale, off, win)
    f = 1.0 if keep is None else keep.astype(np.float64) / (1.0 - float(np.float32(p)))
    wd = bf16(w * f)
    o = bf16(wd @ v)
    dv = bf16(wd.T @ do)
    ds = bf16(w * ((do @ v.T) * f - (do * o).sum(axis=1, keepdims=True)))
    return o, bf16(sc * ds @ k), bf16(sc * ds.T @ q), dv


@pytest.mark.parametrize("Tq,Tk,off,win,p,D", [
    (40, 40, 0, 0, 0.0, 16),
    (33, 50, 17, 0, 0.4, 32),
    (60, 60, 0, 9, 0.25, 16),
    (25, 30, -3, 0, 0.1, 8),
])
def test_bound_contains_the_rounded_computation(Tq, Tk, off, win, p, D):
    B, H = 1, 2
    T = max(Tq, Tk)
    full = W.make_inputs(B, H, T, D, "f32", seed=Tq + D, recipe="iid")
    inp = dict(full)
    for n in ("q", "do"):
        inp[n] = full[n][:, :, T - Tq:].contiguous()
    for n in ("k", "v"):
        inp[n] = full[n][:, :, :Tk].contiguous()
    seed, stream = 1234 + Tq, 5
    bound = rounding_bound(inp, off, win, p, seed, stream)
    q, k, v, do = (inp[n].to(torch.float64).numpy() for n in ("q", "k", "v", "do"))
    for b in range(B):
        for h in range(H):
            keep = philox.keep_mask(b * H + h, Tq, Tk, p, seed, stream) if p > 0 else None
            args = (q[b, h], k[b, h], v[b, h])
            o, _ = A.forward_head(*args, inp["scale"], off, win, keep, p)
            dq, dk, dv = A.backward_head(*args, do[b, h], inp["scale"], off, win, keep, p)
            got = rounded_head(*args, do[b, h], inp["scale"], off, win, keep, p)
            for name, exact, r in zip(("o", "dq", "dk", "dv"), (o, dq, dk, dv), got):
                err = np.abs(r - exact)
                bd = bound[name][b, h]
                assert (err <= bd * (1 + 1e-9) + 1e-12).all(), (
                    name, float(err.max()), float(bd[np.unravel_index(np.argmax(err - bd), err.shape)]))
