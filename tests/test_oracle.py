"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something that is not the oracle: the
pure-Python loop formulation, the lecture's averaging special case computed
in other ways, hand-derived closed forms and worked values, invariants that
follow from the definition, central finite differences, and the float64
scaled-dot-product-attention routine of the PyTorch CPU build.  Together they
are chosen so that a plausible slip in the oracle (a dropped scale, a mask in
the wrong direction, an excluded diagonal, a softmax over the wrong axis, a
transposed operand in the backward, a wrong log base in lse) fails at least
one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return float(np.float32(x))


def randn(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def inputs(B, H, T, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, T, D)) for _ in range(4)]


# --------------------------------------------------------------------------
# 1. Brute-force scalar loops agree with the vectorised definition.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("D", [1, 2, 4])
def test_bruteforce_agrees(T, D):
    q, k, v, do = inputs(2, 2, T, D, seed=100 * T + D)
    sc = f32(1.0 / math.sqrt(D))
    o, lse = A.forward(q, k, v, sc)
    dq, dk, dv = A.backward(q, k, v, do, sc)
    bo, blse = BF.forward(q.tolist(), k.tolist(), v.tolist(), sc)
    bdq, bdk, bdv = BF.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), sc)
    for ours, ref in ((o, bo), (lse, blse), (dq, bdq), (dk, bdk), (dv, bdv)):
        np.testing.assert_allclose(ours, np.array(ref), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# 2. The lecture's averaging special case (Q = 0), three other formulations.
# --------------------------------------------------------------------------

def _version1_loops(v):
    # "version 1: averaging past context with for loops"
    T, D = v.shape
    out = np.zeros((T, D))
    for t in range(T):
        prev = v[: t + 1]
        out[t] = prev.sum(axis=0) / (t + 1)
    return out


def _version2_tril_matmul(v):
    # "version 2: using matrix multiply" with a row-normalised lower triangle
    T = v.shape[0]
    wei = np.tril(np.ones((T, T)))
    wei = wei / wei.sum(axis=1, keepdims=True)
    return wei @ v


def _version3_weights(T):
    # "version 3: adding softmax": zeros, future filled with -inf, softmax
    wei = np.zeros((T, T))
    wei[np.triu(np.ones((T, T), dtype=bool), 1)] = -np.inf
    wei = np.exp(wei - wei.max(axis=1, keepdims=True))
    return wei / wei.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("T", [1, 2, 7, 33])
def test_zero_query_is_prefix_mean(T):
    D = 3
    _, k, v, do = inputs(1, 1, T, D, seed=T)
    q = np.zeros_like(k)
    sc = 0.5
    o, lse = A.forward(q, k, v, sc)
    np.testing.assert_allclose(o[0, 0], _version1_loops(v[0, 0]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, 0], _version2_tril_matmul(v[0, 0]), rtol=0, atol=1e-13)
    p = A.probabilities(q[0, 0], k[0, 0], sc)
    np.testing.assert_allclose(p, _version3_weights(T), rtol=0, atol=1e-15)
    # lse closed form: log of (i + 1) equal terms exp(0)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, T + 1)), rtol=0, atol=1e-14)
    # dV_j = sum_{i >= j} dO_i / (i + 1)
    _, dk, dv = A.backward(q, k, v, do, sc)
    want = np.zeros((T, D))
    for j in range(T):
        for i in range(j, T):
            want[j] += do[0, 0, i] / (i + 1)
    np.testing.assert_allclose(dv[0, 0], want, rtol=0, atol=1e-13)
    assert np.all(dk == 0.0)


def test_golden_prefix_mean_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "prefix_mean_T4.json")))
    T, D = g["T"], g["D"]
    k = np.array(g["k"]).reshape(1, 1, T, D)
    v = np.array(g["v"]).reshape(1, 1, T, D)
    do = np.array(g["do"]).reshape(1, 1, T, D)
    q = np.zeros_like(k)
    o, lse = A.forward(q, k, v, g["scale"])
    dq, dk, dv = A.backward(q, k, v, do, g["scale"])
    np.testing.assert_allclose(o[0, 0], np.array(g["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.array(g["lse"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0], np.array(g["dv"]), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(dk[0, 0], np.array(g["dk"]))


# --------------------------------------------------------------------------
# 3. Hand-derived closed forms.
# --------------------------------------------------------------------------

def test_closed_form_two_tokens_one_dim():
    """T = 2, D = 1 worked by hand.

    Row 0 sees only key 0: o0 = v0, lse0 = s q0 k0.  Row 1 sees keys 0 and 1
    with a = s q1 k0, b = s q1 k1 and weight p = e^a / (e^a + e^b) on key 0:
    o1 = p v0 + (1 - p) v1, lse1 = log(e^a + e^b).  For L = do0 o0 + do1 o1:
      dv0 = do0 + do1 p,  dv1 = do1 (1 - p),  dq0 = 0,
      g   = do1 p (1 - p) (v0 - v1),
      dq1 = g s (k0 - k1),  dk0 = g s q1,  dk1 = -g s q1.
    """
    q0, q1, k0, k1, v0, v1, do0, do1 = 0.3, -1.7, 0.9, 2.2, 1.5, -0.5, 0.8, -1.1
    s = 0.75
    a, b = s * q1 * k0, s * q1 * k1
    p = math.exp(a) / (math.exp(a) + math.exp(b))
    g = do1 * p * (1 - p) * (v0 - v1)
    want = {
        "o": [v0, p * v0 + (1 - p) * v1],
        "lse": [s * q0 * k0, math.log(math.exp(a) + math.exp(b))],
        "dq": [0.0, g * s * (k0 - k1)],
        "dk": [g * s * q1, -g * s * q1],
        "dv": [do0 + do1 * p, do1 * (1 - p)],
    }
    sh = (1, 1, 2, 1)
    q = np.array([q0, q1]).reshape(sh)
    k = np.array([k0, k1]).reshape(sh)
    v = np.array([v0, v1]).reshape(sh)
    do = np.array([do0, do1]).reshape(sh)
    o, lse = A.forward(q, k, v, s)
    dq, dk, dv = A.backward(q, k, v, do, s)
    got = {"o": o.ravel(), "lse": lse.ravel(), "dq": dq.ravel(),
           "dk": dk.ravel(), "dv": dv.ravel()}
    for name in want:
        np.testing.assert_allclose(got[name], want[name], rtol=0, atol=1e-15,
                                   err_msg=name)


def test_single_token():
    q, k, v, do = inputs(2, 3, 1, 5, seed=7)
    sc = 0.125
    o, lse = A.forward(q, k, v, sc)
    dq, dk, dv = A.backward(q, k, v, do, sc)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, sc * (q * k).sum(-1), rtol=0, atol=1e-14)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, do)


def test_first_token_outputs_its_value_exactly():
    q, k, v, do = inputs(2, 2, 17, 8, seed=3)
    o, _ = A.forward(q, k, v, 0.35)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    dq, _, _ = A.backward(q, k, v, do, 0.35)
    np.testing.assert_array_equal(dq[:, :, 0], 0.0)


# --------------------------------------------------------------------------
# 4. Invariants of the definition.
# --------------------------------------------------------------------------

def test_probabilities_rows_and_mask():
    q, k, _, _ = inputs(1, 1, 40, 6, seed=11)
    p = A.probabilities(q[0, 0], k[0, 0], 0.4)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(p[np.triu(np.ones_like(p, dtype=bool), 1)] == 0.0)
    assert np.all(p[np.tril(np.ones_like(p, dtype=bool))] > 0.0)


def test_causality():
    """Changing keys/values at positions after i leaves o_i unchanged."""
    q, k, v, _ = inputs(1, 2, 24, 4, seed=5)
    o, lse = A.forward(q, k, v, 0.5)
    cut = 10
    k2, v2 = k.copy(), v.copy()
    k2[:, :, cut + 1:] += 3.0
    v2[:, :, cut + 1:] -= 7.0
    o2, lse2 = A.forward(q, k2, v2, 0.5)
    np.testing.assert_array_equal(o[:, :, : cut + 1], o2[:, :, : cut + 1])
    np.testing.assert_array_equal(lse[:, :, : cut + 1], lse2[:, :, : cut + 1])
    assert not np.allclose(o[:, :, cut + 1:], o2[:, :, cut + 1:])


def test_batch_and_head_independence():
    q, k, v, _ = inputs(3, 2, 12, 4, seed=9)
    o, _ = A.forward(q, k, v, 0.5)
    q2 = q.copy()
    q2[1, 0] += 1.0
    o2, _ = A.forward(q2, k, v, 0.5)
    mask = np.ones((3, 2), dtype=bool)
    mask[1, 0] = False
    np.testing.assert_array_equal(o[mask], o2[mask])
    # per-head loop (exercise EX1) equals the batched call
    for b in range(3):
        for h in range(2):
            oh, _ = A.forward_head(q[b, h], k[b, h], v[b, h], 0.5)
            np.testing.assert_array_equal(oh, o[b, h])


def test_shift_invariance():
    q, k, v, _ = inputs(1, 1, 20, 5, seed=21)
    o, _ = A.forward(q, k, v, 0.5)
    u = randn((5,), 1)
    c = randn((5,), 2)
    o_k, _ = A.forward(q, k + u, v, 0.5)   # adds q_i . u to every score of row i
    o_v, _ = A.forward(q, k, v + c, 0.5)   # weights sum to one
    np.testing.assert_allclose(o_k, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_v, o + c, rtol=0, atol=1e-12)


def test_gradient_sums():
    q, k, v, do = inputs(2, 2, 30, 6, seed=13)
    dq, dk, dv = A.backward(q, k, v, do, 0.3)
    # rows of dS sum to zero, so do the key gradients over positions
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    # rows of P sum to one, so sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0, atol=1e-12)


def test_linear_in_output_gradient():
    q, k, v, do1 = inputs(1, 2, 15, 4, seed=17)
    do2 = randn(do1.shape, 18)
    a, b = 0.7, -1.9
    g1 = A.backward(q, k, v, do1, 0.5)
    g2 = A.backward(q, k, v, do2, 0.5)
    g = A.backward(q, k, v, a * do1 + b * do2, 0.5)
    for x, x1, x2 in zip(g, g1, g2):
        np.testing.assert_allclose(x, a * x1 + b * x2, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# 5. Finite differences of L = sum(O * dO).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("D", [2, 4])
def test_finite_differences(T, D):
    q, k, v, do = inputs(1, 2, T, D, seed=31 * T + D)
    sc = f32(1.0 / math.sqrt(D))
    grads = A.backward(q, k, v, do, sc)
    h = 1e-6

    def loss(qq, kk, vv):
        o, _ = A.forward(qq, kk, vv, sc)
        return float((o * do).sum())

    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        base = [q, k, v]
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        scale_ref = max(1.0, np.abs(g).max())
        np.testing.assert_allclose(fd, g, rtol=0, atol=1e-7 * scale_ref)


# --------------------------------------------------------------------------
# 6. Library cross-check: PyTorch's float64 CPU attention routine.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,D", [(1, 4), (9, 8), (64, 16), (130, 32)])
def test_matches_torch_sdpa_float64(T, D):
    q, k, v, do = inputs(2, 3, T, D, seed=T + D)
    sc = f32(1.0 / math.sqrt(D))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=sc)
    to.backward(torch.tensor(do))
    o, _ = A.forward(q, k, v, sc)
    dq, dk, dv = A.backward(q, k, v, do, sc)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_selected_heads_only():
    q, k, v, do = inputs(2, 3, 10, 4, seed=1)
    o_all, lse_all = A.forward(q, k, v, 0.5)
    o_sel, lse_sel = A.forward(q, k, v, 0.5, heads=[(1, 2), (0, 0)])
    np.testing.assert_array_equal(o_sel[1, 2], o_all[1, 2])
    np.testing.assert_array_equal(lse_sel[0, 0], lse_all[0, 0])
    assert np.isnan(o_sel[0, 1]).all()


def test_rounding_variant_is_close_to_the_definition():
    """The bf16-rounding diagnostic differs from the float64 definition by a
    few bf16 units, and not at all when every quantity is representable."""
    from oracle import rounding as R
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((12, 8)) * s for s in (0.5, 0.5, 1.0, 0.01))
    o, _ = A.forward_head(q, k, v, 0.375)
    ob = R.forward_head(q, k, v, 0.375)
    assert 0 < np.abs(ob - o).max() < 4 * 2.0 ** -8 * np.abs(o).max()
    g = A.backward_head(q, k, v, do, 0.375)
    gb = R.backward_head(q, k, v, do, 0.375)
    for x, y in zip(g, gb):
        assert np.linalg.norm(x - y) <= 2e-2 * np.linalg.norm(x)
    # one key per row (T = 1): P = 1 is exact, so O = bf16(V)
    v1 = R.bf16(v[:1])
    np.testing.assert_array_equal(R.forward_head(q[:1], k[:1], v1, 0.375), v1)
