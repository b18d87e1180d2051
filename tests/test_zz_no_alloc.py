"""GPU check of the no-allocation backward entry point: gptattn_bwd_noalloc
(called through the C ABI) against gptattn_bwd on the same inputs, on two
calls in a row, the second with a smaller problem than the first (the
scratch array keeps the first call's values; nothing may leak into the
second).  The kernels are the same, so the results must be bit-identical."""

import ctypes

import pytest
import torch

import causal_self_attention_gptattn_amd as G
from causal_self_attention_gptattn_amd import workloads as W

from gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("D", [64, 128])
def test_noalloc_equals_workspace_backward_twice(D):
    dev = need_gpu()
    lib = G.library()
    for B, H, T in ((3, 5, 700), (1, 3, 129)):
        say("no-alloc backward", B, H, T, D)
        inp = W.make_inputs(B, H, T, D, "bf16", seed=T + D)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        sc = inp["scale"]
        o, lse = G.fwd(q, k, v, sc)
        ref = G.bwd(q, k, v, o, do, lse, sc)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        rc = lib.gptattn_bwd_noalloc(_p(q), _p(k), _p(v), _p(o), _p(do), _p(lse),
                                     *[_p(t) for t in got], B, H, T, D, sc,
                                     ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        assert rc == 0, G.status_string(rc)
        torch.cuda.synchronize(dev)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), "%s differs (B=%d H=%d T=%d D=%d)" % (name, B, H, T, D)
    # the Python wrapper of the same entry point
    g2 = G.bwd_noalloc(q, k, v, o, do, lse, sc)
    torch.cuda.synchronize(dev)
    for a, b in zip(g2, ref):
        assert torch.equal(a, b)
