"""Pins for the oracle's generalised visibility: a causal offset (Tq != Tk,
queries appended to a context) and a local window (banded attention).

Each check compares the oracle with something that is not the oracle: the
pure-Python loops, closed forms (window 1), the plain causal oracle on a
larger problem (prefix consistency), PyTorch's float64 attention routine with
an explicit mask, and finite differences.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import bruteforce as BF


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CASES = [  # (Tq, Tk, offset, window)
    (5, 5, 0, 2), (5, 5, 0, 1), (3, 7, 4, 0), (3, 7, 4, 3), (1, 8, 7, 0), (1, 8, 7, 4),
    (6, 4, -2, 0), (4, 6, 0, 0), (7, 7, 0, 30), (6, 3, -3, 2),
]


@pytest.mark.parametrize("Tq,Tk,off,win", CASES)
def test_bruteforce_agrees(Tq, Tk, off, win):
    D = 3
    q = rnd((2, 2, Tq, D), 1)
    k = rnd((2, 2, Tk, D), 2)
    v = rnd((2, 2, Tk, D), 3)
    do = rnd((2, 2, Tq, D), 4)
    sc = 0.625
    o, lse = A.forward(q, k, v, sc, offset=off, window=win)
    g = A.backward(q, k, v, do, sc, offset=off, window=win)
    bo, blse = BF.forward(q.tolist(), k.tolist(), v.tolist(), sc, off, win)
    bg = BF.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), sc, off, win)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(np.array(blse)))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], np.array(blse)[fin], rtol=0, atol=1e-12)
    for x, y in zip(g, bg):
        np.testing.assert_allclose(x, np.array(y), rtol=0, atol=1e-12)


def test_rows_that_see_nothing():
    # offset -2: queries 0 and 1 have no key at or before them
    q, k, v, do = (rnd((1, 1, 4, 2), s) for s in range(4))
    o, lse = A.forward(q, k, v, 0.5, offset=-2)
    dq, dk, dv = A.backward(q, k, v, do, 0.5, offset=-2)
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(dq[0, 0, :2] == 0)
    np.testing.assert_array_equal(o[0, 0, 2], v[0, 0, 0])   # row 2 sees only key 0
    assert np.isfinite(lse[0, 0, 2:]).all()


@pytest.mark.parametrize("off", [0, 3])
def test_window_one_is_the_diagonal_key(off):
    """With window 1 each query sees exactly key i + offset: O_i = V_{i+off},
    lse_i = scale q_i . k_{i+off}; no gradient reaches Q or K, and
    dV_{i+off} = dO_i."""
    Tq, D, sc = 6, 4, 0.375
    Tk = Tq + off
    q, do = rnd((1, 1, Tq, D), 1), rnd((1, 1, Tq, D), 4)
    k, v = rnd((1, 1, Tk, D), 2), rnd((1, 1, Tk, D), 3)
    o, lse = A.forward(q, k, v, sc, offset=off, window=1)
    dq, dk, dv = A.backward(q, k, v, do, sc, offset=off, window=1)
    np.testing.assert_array_equal(o[0, 0], v[0, 0, off:])
    np.testing.assert_allclose(lse[0, 0], sc * (q[0, 0] * k[0, 0, off:]).sum(-1), rtol=0,
                               atol=1e-14)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv[0, 0, off:], do[0, 0])
    np.testing.assert_array_equal(dv[0, 0, :off], 0)


def test_wide_window_is_plain_causal():
    q, k, v, do = (rnd((2, 3, 9, 4), s) for s in range(4))
    a = A.forward(q, k, v, 0.375, window=9)
    b = A.forward(q, k, v, 0.375)
    np.testing.assert_array_equal(a[0], b[0])
    for x, y in zip(A.backward(q, k, v, do, 0.375, window=50), A.backward(q, k, v, do, 0.375)):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("win", [0, 3])
def test_prefix_consistency(win):
    """Appending Tq queries to a Tk-position context (offset Tk - Tq) gives
    the last Tq rows of the full causal problem over Tk positions."""
    Tk, Tq, D, sc = 11, 4, 5, 0.375
    qf = rnd((1, 2, Tk, D), 1)
    k, v = rnd((1, 2, Tk, D), 2), rnd((1, 2, Tk, D), 3)
    dof = rnd((1, 2, Tk, D), 4)
    dof[:, :, : Tk - Tq] = 0.0   # only the appended rows carry a gradient
    q, do = qf[:, :, Tk - Tq:], dof[:, :, Tk - Tq:]
    o_full, l_full = A.forward(qf, k, v, sc, window=win)
    o, l = A.forward(q, k, v, sc, offset=Tk - Tq, window=win)
    np.testing.assert_allclose(o, o_full[:, :, Tk - Tq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_full[:, :, Tk - Tq:], rtol=0, atol=1e-13)
    gf = A.backward(qf, k, v, dof, sc, window=win)
    g = A.backward(q, k, v, do, sc, offset=Tk - Tq, window=win)
    np.testing.assert_allclose(g[0], gf[0][:, :, Tk - Tq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g[1], gf[1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g[2], gf[2], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Tq,Tk,off,win", [(9, 9, 0, 3), (5, 12, 7, 4), (12, 12, 0, 1),
                                           (8, 16, 8, 0)])
def test_matches_torch_sdpa_with_mask(Tq, Tk, off, win):
    D = 8
    q, do = rnd((2, 2, Tq, D), 1), rnd((2, 2, Tq, D), 4)
    k, v = rnd((2, 2, Tk, D), 2), rnd((2, 2, Tk, D), 3)
    sc = float(np.float32(1 / math.sqrt(D)))
    mask = torch.tensor(A.visible(Tq, Tk, off, win))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sc)
    to.backward(torch.tensor(do))
    o, _ = A.forward(q, k, v, sc, offset=off, window=win)
    dq, dk, dv = A.backward(q, k, v, do, sc, offset=off, window=win)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_finite_differences_banded_offset():
    Tq, Tk, off, win, D, sc = 4, 6, 2, 3, 3, 0.6875
    q, do = rnd((1, 1, Tq, D), 1), rnd((1, 1, Tq, D), 4)
    k, v = rnd((1, 1, Tk, D), 2), rnd((1, 1, Tk, D), 3)
    grads = A.backward(q, k, v, do, sc, offset=off, window=win)
    h = 1e-6

    def loss(qq, kk, vv):
        return float((A.forward(qq, kk, vv, sc, offset=off, window=win)[0] * do).sum())

    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            plus, minus = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(fd, g, rtol=0, atol=1e-7 * max(1.0, np.abs(g).max()))
