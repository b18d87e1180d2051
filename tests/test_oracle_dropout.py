"""Pins for the oracle's attention dropout and its counter-based generator.

* Philox4x32-10 against the known-answer vectors published with the
  generator's reference implementation (Random123, the library accompanying
  Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).
* The keep mask: drop rate within binomial bounds, independence of heads and
  streams, and its word mapping against single scalar generator calls.
* Dropout arithmetic: the pure-Python loops with the same mask, PyTorch
  float64 autograd through an explicitly masked softmax, finite differences
  with the mask held fixed, p = 0 reducing to plain attention, and the
  dropped-out output being unbiased over many seeds.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import bruteforce as BF
from oracle import philox as P


KAT = [  # (counter, key) -> output, Random123 known-answer vectors for philox4x32-10
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = P.philox4x32_10(*[np.uint64(c) for c in ctr], key[0], key[1])
    assert tuple(int(g) for g in got) == out


def test_threshold():
    assert P.threshold(0.0) == 0
    assert P.threshold(0.5) == 2 ** 15
    assert P.threshold(0.25) == 2 ** 14
    p = float(np.float32(0.1))
    assert P.threshold(0.1) == math.ceil(p * 2 ** 16)
    # the largest float32 below 1 drops every weight
    assert P.threshold(float(np.nextafter(np.float32(1), np.float32(0)))) == 2 ** 16


@pytest.mark.parametrize("p", [0.1, 0.3, 0.5, 0.9, 1e-5, 0.999])
def test_keep_scale_averages_to_one_over_all_draws(p):
    """The kept-weight factor is the inverse of the keep probability the
    16-bit threshold realises: over the 2^16 equally likely draws, the mean of
    keep * scale is 1 (the dropped-out weights are unbiased).  With the
    nominal 1 / (1 - p) instead, p = 0.1 (thr rounded up from 6553.6) misses
    by 6e-6."""
    thr = P.threshold(p)
    draws = np.arange(2 ** 16)
    mean = ((draws >= thr) * P.keep_scale(p)).mean()
    assert abs(mean - 1.0) <= 1e-15
    assert P.keep_scale(p) == 2.0 ** 16 / (2 ** 16 - thr)
    # the scalar-loop twin computes the same factor on its own
    assert BF._keep_scale(p) == P.keep_scale(p)


def test_keep_scale_when_everything_is_dropped():
    p = float(np.nextafter(np.float32(1), np.float32(0)))
    assert P.threshold(p) == 2 ** 16 and P.keep_scale(p) == 0.0
    assert BF._keep_scale(p) == 0.0


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_drop_rate_is_binomial(p):
    m = P.keep_mask(3, 256, 512, p, seed=1234, stream=7)
    n = m.size
    dropped = n - m.sum()
    sd = math.sqrt(n * p * (1 - p))
    assert abs(dropped - n * p) < 5 * sd


def test_masks_differ_across_heads_streams_seeds():
    base = P.keep_mask(0, 64, 64, 0.5, seed=1, stream=0)
    for other in (P.keep_mask(1, 64, 64, 0.5, seed=1, stream=0),
                  P.keep_mask(0, 64, 64, 0.5, seed=1, stream=1),
                  P.keep_mask(0, 64, 64, 0.5, seed=2, stream=0),
                  P.keep_mask(0, 64, 64, 0.5, seed=1 + (1 << 32), stream=0)):
        agree = (base == other).mean()
        assert 0.4 < agree < 0.6


def test_mask_word_mapping():
    """Element (i, j) is the 16-bit half i % 2 (low for even i) of word j % 4
    of the call on counter (j // 4, i // 2, n, stream)."""
    n, seed, stream, p = 5, 0x123456789ABCDEF, 3, 0.3
    m = P.keep_mask(n, 9, 13, p, seed, stream)
    thr = P.threshold(p)
    for i in range(9):
        for j in range(13):
            w = P.philox4x32_10(np.uint64(j // 4), np.uint64(i // 2), np.uint64(n),
                                np.uint64(stream), seed & 0xFFFFFFFF, seed >> 32)
            x = (int(w[j % 4]) >> (16 * (i % 2))) & 0xFFFF
            assert m[i, j] == (x >= thr)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def masks(B, H, Tq, Tk, p, seed):
    return np.stack([np.stack([P.keep_mask(b * H + h, Tq, Tk, p, seed) for h in range(H)])
                     for b in range(B)])


@pytest.mark.parametrize("Tq,Tk,off,win", [(6, 6, 0, 0), (4, 7, 3, 0), (6, 6, 0, 3)])
def test_bruteforce_agrees_with_dropout(Tq, Tk, off, win):
    B, H, D, p, seed, sc = 2, 2, 3, 0.3, 77, 0.625
    q, do = rnd((B, H, Tq, D), 1), rnd((B, H, Tq, D), 4)
    k, v = rnd((B, H, Tk, D), 2), rnd((B, H, Tk, D), 3)
    o, lse = A.forward(q, k, v, sc, offset=off, window=win, dropout=p, seed=seed)
    g = A.backward(q, k, v, do, sc, offset=off, window=win, dropout=p, seed=seed)
    keep = masks(B, H, Tq, Tk, p, seed).tolist()
    p32 = float(np.float32(p))  # the library takes p as a float32
    bo, blse = BF.forward(q.tolist(), k.tolist(), v.tolist(), sc, off, win, keep, p32)
    bg = BF.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), sc, off, win, keep, p32)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(blse), rtol=0, atol=1e-12)
    for x, y in zip(g, bg):
        np.testing.assert_allclose(x, np.array(y), rtol=0, atol=1e-12)


def test_torch_autograd_with_explicit_mask():
    B, H, T, D, p, seed, sc = 1, 3, 10, 4, 0.25, 5, 0.375
    q, k, v, do = (rnd((B, H, T, D), s) for s in range(4))
    keep = masks(B, H, T, T, p, seed)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = sc * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    w = torch.softmax(s, dim=-1) * torch.tensor(keep, dtype=torch.float64) / (1 - float(np.float32(p)))
    to = w @ tv
    to.backward(torch.tensor(do))
    o, _ = A.forward(q, k, v, sc, dropout=p, seed=seed)
    dq, dk, dv = A.backward(q, k, v, do, sc, dropout=p, seed=seed)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    for a, b in zip((dq, dk, dv), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)


def test_finite_differences_with_fixed_mask():
    T, D, p, sc = 5, 3, 0.4, 0.6875
    q, k, v, do = (rnd((1, 1, T, D), s) for s in range(4))
    keep = P.keep_mask(0, T, T, p, seed=9)
    grads = A.backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], sc, keep=keep, p=p)
    h = 1e-6

    def loss(qq, kk, vv):
        return float((A.forward_head(qq, kk, vv, sc, keep=keep, p=p)[0] * do[0, 0]).sum())

    base = [q[0, 0], k[0, 0], v[0, 0]]
    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(fd, g, rtol=0, atol=1e-7 * max(1.0, np.abs(g).max()))


def test_zero_probability_is_plain_attention():
    q, k, v, do = (rnd((2, 2, 7, 3), s) for s in range(4))
    a = A.forward(q, k, v, 0.5, dropout=0.0, seed=3)
    b = A.forward(q, k, v, 0.5)
    np.testing.assert_array_equal(a[0], b[0])
    for x, y in zip(A.backward(q, k, v, do, 0.5, dropout=0.0, seed=3),
                    A.backward(q, k, v, do, 0.5)):
        np.testing.assert_array_equal(x, y)


def test_dropout_is_unbiased():
    """Averaged over many seeds, O with dropout approaches O without it."""
    T, D, p = 12, 4, 0.3
    q, k, v = (rnd((1, 1, T, D), s) for s in range(3))
    ref, _ = A.forward(q, k, v, 0.5)
    acc = np.zeros_like(ref)
    n = 400
    for seed in range(n):
        acc += A.forward(q, k, v, 0.5, dropout=p, seed=seed)[0]
    mean = acc / n
    # per element: the weights' dropout noise has variance p/(1-p) P^2 per term
    assert np.abs(mean - ref).max() < 0.15
    assert np.abs(mean - ref).mean() < 0.03
