"""Pins for oracle.rounding, the diagnostic that repeats the float64
definition with the bf16 kernels' storage roundings (P before P.V and
P^T.dO, dS before the dQ and dK products, every output once).

* Its rounding function is checked against an independent one written from
  the bfloat16 format (8 significant bits, round to nearest, ties to even),
  applied to the float32 value, which is what the kernels round.
* A scalar-loop twin written here, with that independent rounding at the
  points listed above, must reproduce the diagnostic bit for bit, and the
  same twin with any one rounding left out must not: so the comparison
  would catch a dropped or misplaced rounding.
* A hand-worked two-token case where rounding P makes two nearly equal
  weights cancel exactly.
"""

import math

import numpy as np

from oracle import attention as A
from oracle import rounding as R


def bf16_ref(x):
    """float64 -> float32 (nearest even) -> bfloat16 (nearest even), from the
    format: keep 8 significant bits of the float32 value."""
    x32 = float(np.float32(x))
    if x32 == 0.0 or not math.isfinite(x32):
        return x32
    m, e = math.frexp(x32)  # x32 = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)  # round(): ties to even


def test_rounding_function_matches_the_format():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    got = R.bf16(x)
    assert all(got[i] == bf16_ref(x[i]) for i in range(len(x)))
    # ties go to the even neighbour; just past a tie, away from it
    one = 1.0
    assert R.bf16(np.array([one + 2.0 ** -8]))[0] == 1.0
    assert R.bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert R.bf16(np.array([one + 2.0 ** -8 + 2.0 ** -20]))[0] == 1.0 + 2.0 ** -7
    assert R.bf16(np.array([-(one + 2.0 ** -8)]))[0] == -1.0


def twin(q, k, v, do, scale, skip=()):
    """Scalar loops over one causal head: (O, dQ, dK, dV) with bf16 rounding
    of P, dS and the outputs unless named in `skip`."""
    T, D = len(q), len(q[0])
    sc = float(np.float32(scale))
    r = {n: (lambda x: x) if n in skip else bf16_ref for n in ("p", "ds", "out")}
    P = [[0.0] * T for _ in range(T)]
    for i in range(T):
        s = [sc * sum(q[i][d] * k[j][d] for d in range(D)) for j in range(i + 1)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l_ = sum(e)
        for j in range(i + 1):
            P[i][j] = e[j] / l_
    O = [[r["out"](sum(r["p"](P[i][j]) * v[j][d] for j in range(i + 1))) for d in range(D)]
         for i in range(T)]
    dV = [[r["out"](sum(r["p"](P[i][j]) * do[i][d] for i in range(j, T))) for d in range(D)]
          for j in range(T)]
    row = [sum(do[i][d] * O[i][d] for d in range(D)) for i in range(T)]
    dS = [[r["ds"](P[i][j] * (sum(do[i][d] * v[j][d] for d in range(D)) - row[i]))
           if j <= i else 0.0 for j in range(T)] for i in range(T)]
    dQ = [[r["out"](sc * sum(dS[i][j] * k[j][d] for j in range(i + 1))) for d in range(D)]
          for i in range(T)]
    dK = [[r["out"](sc * sum(dS[i][j] * q[i][d] for i in range(j, T))) for d in range(D)]
          for j in range(T)]
    return [np.array(x) for x in (O, dQ, dK, dV)]


def diagnostic(q, k, v, do, scale):
    o = R.forward_head(q, k, v, scale)
    dq, dk, dv = R.backward_head(q, k, v, do, scale)
    return [o, dq, dk, dv]


def case(seed, T=9, D=5):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, D)) * s for s in (0.8, 0.8, 1.0, 0.3)]


def test_diagnostic_matches_the_scalar_twin_bit_for_bit():
    for seed in range(4):
        q, k, v, do = case(seed)
        for name, a, b in zip(("o", "dq", "dk", "dv"), diagnostic(q, k, v, do, 0.4),
                              twin(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.4)):
            np.testing.assert_array_equal(a, b, err_msg="%s seed %d" % (name, seed))


def test_every_rounding_is_seen_by_the_comparison():
    """Leaving any one rounding out of the twin changes its result on these
    inputs, so the bit-for-bit comparison above pins each of them."""
    q, k, v, do = case(0)
    ref = diagnostic(q, k, v, do, 0.4)
    for skip, affected in ((("p",), ("o", "dv")), (("ds",), ("dq", "dk")),
                           (("out",), ("o", "dq", "dk", "dv"))):
        alt = dict(zip(("o", "dq", "dk", "dv"),
                       twin(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.4, skip)))
        for name in affected:
            assert not np.array_equal(alt[name], ref[("o", "dq", "dk", "dv").index(name)]), \
                (skip, name)


def test_rounded_weights_cancel_in_a_two_token_case():
    """Query 1 sees keys 0 and 1 with scores 1e-3 and 0 (scale 1), so its
    weights are 0.50025 and 0.49975; both round to 0.5 in bf16.  With
    v_0 = -v_1 the rounded output is exactly 0, where the definition gives
    5e-4; with dO_0 = -dO_1 / 2, dV_0 = dO_0 + 0.5 dO_1 = 0 likewise."""
    d = 1e-3
    q = np.array([[1.0, 0.0], [1.0, 0.0]])
    k = np.array([[d, 0.0], [0.0, 0.0]])
    v = np.array([[1.0, 0.0], [-1.0, 0.0]])
    do = np.array([[-0.5, 0.0], [1.0, 0.0]])
    o_def, _ = A.forward_head(q, k, v, 1.0)
    assert abs(o_def[1, 0] - math.tanh(d / 2)) < 1e-15   # p0 - p1 = tanh(d / 2)
    assert R.forward_head(q, k, v, 1.0)[1, 0] == 0.0
    dv_def = A.backward_head(q, k, v, do, 1.0)[2]
    assert abs(dv_def[0, 0] - (-0.5 + 1 / (1 + math.exp(-d)))) < 1e-15
    assert R.backward_head(q, k, v, do, 1.0)[2][0, 0] == 0.0


def test_outputs_are_bf16_values():
    q, k, v, do = case(5, T=16, D=8)
    for x in diagnostic(q, k, v, do, 0.35):
        np.testing.assert_array_equal(x, R.bf16(x))
