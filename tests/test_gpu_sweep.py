"""Seeded sweep of the strided entry points against the float64 oracle.

A hundred and twenty configurations drawn from a fixed seed cover
combinations the hand-picked cases do not: both precisions and every
compiled head size; Tq and Tk from 1 to 600 (including Tq > Tk); causal
offsets that leave rows without keys or let every row see everything;
banded windows; dense, [B, T, H, D]-transposed and packed [B, T, 3C]
layouts; and dropout.  A long sequence (16384 positions) is checked on
sampled row blocks of the forward pass, which the oracle computes exactly
by shifting the causal offset.
"""

import numpy as np
import pytest
import torch

import causal_self_attention_gptattn_amd as G
from causal_self_attention_gptattn_amd import workloads as W

from gpu_helpers import compare, need_gpu, rounding_bound, say, to64

pytestmark = pytest.mark.gpu


def draw_configs(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        f32 = rng.random() < 0.3
        D = int(rng.choice([16, 32, 64])) if f32 else int(rng.choice([64, 128]))
        Tk = int(rng.integers(1, 601))
        Tq = int(rng.integers(1, 601)) if rng.random() < 0.5 else Tk
        r = rng.random()
        if r < 0.4:
            off = Tk - Tq                      # queries aligned to the end of the keys
        elif r < 0.6:
            off = 0
        else:
            off = int(rng.integers(-50, Tk + 20))
        win = 0 if rng.random() < 0.6 else int(rng.integers(1, 300))
        layout = str(rng.choice(["dense", "bthd", "packed"]))
        if layout == "packed" and Tq != Tk:
            layout = "bthd"
        drop = 0.0 if rng.random() < 0.7 else float(rng.choice([0.1, 0.4]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        out.append((idx, "f32" if f32 else "bf16", B, H, Tq, Tk, D, off, win, layout, drop))
    return out


def place(inp, layout, dev, dtype):
    """The inputs as views of the requested layout (values unchanged)."""
    q, k, v, do = (inp[n] for n in ("q", "k", "v", "do"))
    if layout == "dense":
        return tuple(t.to(dev) for t in (q, k, v, do)), lambda like: torch.empty_like(like)
    if layout == "bthd":
        views = tuple(t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v, do))

        def alloc(like):
            B, H, T, D = like.shape
            return torch.empty(B, T, H, D, dtype=like.dtype, device=dev).transpose(1, 2)
        return views, alloc
    B, H, T, D = q.shape
    x = torch.cat([t.transpose(1, 2).reshape(B, T, H * D) for t in (q, k, v)], dim=-1)
    qv, kv, vv = G.split_qkv(x.to(dev).contiguous(), H)
    return (qv, kv, vv, do.to(dev)), lambda like: torch.empty_like(like, memory_format=torch.contiguous_format)


@pytest.mark.parametrize("cfg", draw_configs(120), ids=lambda c: "c%03d" % c[0])
def test_sweep(cfg):
    from oracle import attention as A
    dev = need_gpu()
    idx, dtype, B, H, Tq, Tk, D, off, win, layout, drop = cfg
    say("sweep", cfg)
    T = max(Tq, Tk)
    full = W.make_inputs(B, H, T, D, dtype, seed=100 + idx, recipe="iid")
    inp = dict(full)
    for n_ in ("q", "do"):
        inp[n_] = full[n_][:, :, T - Tq:].contiguous()
    for n_ in ("k", "v"):
        inp[n_] = full[n_][:, :, :Tk].contiguous()
    (q, k, v, do), alloc = place(inp, layout, dev, dtype)
    kw = dict(dropout=drop, seed=77 + idx, rng_stream=idx)
    o, lse = G.fwd_ex(q, k, v, inp["scale"], off, win, out=alloc(q), **kw)
    dq, dk, dv = G.bwd_ex(q, k, v, o, do, lse, inp["scale"], off, win, dq=alloc(q), dk=alloc(k),
                          dv=alloc(v), **kw)
    torch.cuda.synchronize()
    got = {"o": to64(o), "lse": to64(lse), "dq": to64(dq), "dk": to64(dk), "dv": to64(dv)}
    qq, kk, vv, dd = (inp[n_].to(torch.float64).numpy() for n_ in ("q", "k", "v", "do"))
    okw = dict(offset=off, window=win, dropout=drop, seed=77 + idx, stream=idx)
    ro, rl = A.forward(qq, kk, vv, inp["scale"], **okw)
    rdq, rdk, rdv = A.backward(qq, kk, vv, dd, inp["scale"], **okw)
    ref = {"o": ro, "lse": rl, "dq": rdq, "dk": rdk, "dv": rdv}
    bound = rounding_bound(inp, off, win, drop, 77 + idx, idx) if dtype == "bf16" else None
    compare(got, ref, dtype, label="sweep %s" % (cfg,), bound=bound)


@pytest.mark.parametrize("D", [64, 128])
def test_long_sequence_forward_rows(D):
    """16384 positions, one head: sampled 64-row blocks of O and lse, each
    computed by the oracle as Tq = 64 queries at offset i0."""
    from oracle import attention as A
    dev = need_gpu()
    T = 16384
    inp = W.make_inputs(1, 1, T, D, "bf16", seed=D, recipe="iid")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = G.fwd(q, k, v, inp["scale"])
    torch.cuda.synchronize()
    o64, l64 = to64(o), to64(lse)
    qq, kk, vv = (inp[n].to(torch.float64).numpy() for n in ("q", "k", "v"))
    for i0 in (0, 4096 - 32, 9000, T - 64):
        ro, rl = A.forward(qq[:, :, i0:i0 + 64], kk[:, :, :i0 + 64], vv[:, :, :i0 + 64],
                           inp["scale"], offset=i0)
        got = {"o": o64[:, :, i0:i0 + 64], "lse": l64[:, :, i0:i0 + 64]}
        err_o = np.abs(got["o"] - ro).max()
        lim = 2e-2 + 2.0 ** -8 * np.abs(ro)
        assert (np.abs(got["o"] - ro) <= lim).all(), "rows %d: O err %.3e" % (i0, err_o)
        assert np.abs(got["lse"] - rl).max() <= 1e-3, "rows %d: lse" % i0
        say("long T=%d D=%d rows %d: O err %.2e" % (T, D, i0, err_o))


@pytest.mark.parametrize("B,H,T,D", [
    (48, 12, 1024, 64),   # 576 heads: 9 rounds of dQ's slots (dQ grouped, forward not)
    (96, 12, 1024, 64),   # 1152 heads: dQ grouped (the D = 64 forward keeps its dealt order)
    (256, 8, 256, 128),   # 2048 heads: 8 rounds of the forward's and dQ's slots, 16 of
                          # dK/dV's (all three grouped)
])
def test_heads_in_groups(B, H, T, D):
    """A problem of eight or more rounds of workgroup slots runs dQ (and, at
    D = 128, the forward and dK/dV) with its heads in groups.  Every output
    of the whole launch must equal, bit for bit, that of the same heads
    launched in batches small enough for the plain order on the same kernels
    (the per-head arithmetic is the same, so any head missed, repeated or
    mixed up by the grouped order shows), and heads at the group edges and
    inside the groups are checked against the oracle."""
    from oracle import attention as A
    dev = need_gpu()
    g = torch.Generator().manual_seed(11)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g).to(torch.bfloat16) for _ in range(4))
    do = (do.float() * 0.01).to(torch.bfloat16)
    sc = W.default_scale(D)
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, do))
    o, lse = G.fwd(qd, kd, vd, sc)
    dq, dk, dv = G.bwd(qd, kd, vd, o, dd, lse, sc)
    torch.cuda.synchronize()
    # the same heads in batches of fewer rounds (plain order), large enough
    # for the persistent dK/dV grid (more 128-key items than compute units)
    step = 16 if D == 64 else 32
    parts = {n_: [] for n_ in ("o", "lse", "dq", "dk", "dv")}
    for b0 in range(0, B, step):
        sl = slice(b0, b0 + step)
        op, lp = G.fwd(qd[sl], kd[sl], vd[sl], sc)
        dqp, dkp, dvp = G.bwd(qd[sl], kd[sl], vd[sl], o[sl], dd[sl], lse[sl], sc)
        for n_, t in (("o", op), ("lse", lp), ("dq", dqp), ("dk", dkp), ("dv", dvp)):
            parts[n_].append(t)
    torch.cuda.synchronize()
    for n_, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(t, torch.cat(parts[n_])), "grouped %s differs from the batched runs" % n_
    N = B * H
    picks = sorted({0, N // 3 - 1, N // 3, N // 2 - 1, N // 2, 2 * N // 3, N - 1, 5 * N // 7})
    for n in picks:
        b, h = divmod(n, H)
        ins = [t[b:b + 1, h:h + 1].double().numpy() for t in (q, k, v, do)]
        ro, rl = A.forward(*ins[:3], sc)
        rq, rk, rv = A.backward(*ins, sc)
        got = {n_: to64(t[b:b + 1, h:h + 1]) for n_, t in
               (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
        compare(got, {"o": ro, "lse": rl, "dq": rq, "dk": rk, "dv": rv}, "bf16",
                label="heads in groups %s head %d" % ((B, H, T, D), n))


def test_many_heads_large_grid():
    """32768 head-problems of 65 positions: a grid of 32768 workgroups per
    launch, every head computed; sampled heads checked against the oracle."""
    from oracle import attention as A
    dev = need_gpu()
    B, H, T, D = 256, 128, 65, 64
    g = torch.Generator().manual_seed(5)
    q, k, v, do = (torch.randn(B, H, T, D, generator=g).to(torch.bfloat16) for _ in range(4))
    do = (do.float() * 0.01).to(torch.bfloat16)
    qd, kd, vd, dd = (t.to(dev) for t in (q, k, v, do))
    o, lse = G.fwd(qd, kd, vd, 0.125)
    dq, dk, dv = G.bwd(qd, kd, vd, o, dd, lse, 0.125)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (37, 101), (255, 127), (128, 64)):
        ro, rl = A.forward(*(t[b:b + 1, h:h + 1].double().numpy() for t in (q, k, v)), 0.125)
        rq, rk, rv = A.backward(*(t[b:b + 1, h:h + 1].double().numpy() for t in (q, k, v, do)),
                                0.125)
        got = {n_: to64(t[b:b + 1, h:h + 1]) for n_, t in
               (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
        compare(got, {"o": ro, "lse": rl, "dq": rq, "dk": rk, "dv": rv}, "bf16",
                label="many heads (%d,%d)" % (b, h))
