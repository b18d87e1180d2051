"""Pure-Python scalar-loop formulation of causal self-attention (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No numpy: nested
lists of Python floats (IEEE double) and ``math.exp``/``math.log``, so it
shares no vectorised primitive with :mod:`oracle.attention`.  Meant for tiny
shapes (T <= 8); cost is O(T^2 D) Python operations per head.

It follows the "Let's build GPT: from scratch, in code, spelled out" lecture
description page: "version 1" walks over the past context with explicit
loops; "version 3" turns masked affinities into weights with a softmax;
"version 4" makes the affinities query-key dot products scaled by
1/sqrt(head_size) (note 6 and the 01:20:05 correction); the 00:57:00
correction fixes that only past and present positions are visible.

Inputs are nested lists indexed ``[b][h][t][d]``; so are the outputs
(``lse`` is ``[b][h][t]``).  The optional ``offset`` and ``window`` select
which keys a query sees exactly as in :func:`oracle.attention.visible`.
``keep`` (nested ``[b][h][i][j]`` booleans) and ``drop`` apply dropout to
the weights: a dropped weight is 0, a kept one is multiplied by the inverse
of the keep probability the 16-bit draws realise, 2^16 / (2^16 - thr) with
thr = ceil(p * 2^16) for the float32 value p of ``drop``.
"""

import math
import struct


def _keys(i, Tk, offset, window):
    """Keys query i may look at: j <= i + offset, and j > i + offset - window
    when a window is set; never the future."""
    hi = min(Tk - 1, i + offset)
    lo = max(0, i + offset - window + 1) if window > 0 else 0
    return list(range(lo, hi + 1))


def _keep_scale(drop):
    """2^16 / (2^16 - thr): a draw x in 0 .. 2^16 - 1 keeps the weight iff
    x >= thr, so 2^16 - thr of the 2^16 draws keep it."""
    p32 = struct.unpack("<f", struct.pack("<f", drop))[0]
    thr = min(math.ceil(p32 * 65536.0), 65536) if p32 > 0 else 0
    return 65536.0 / (65536 - thr) if thr < 65536 else 0.0


def _factor(keep, i, j, drop):
    if keep is None:
        return 1.0
    return _keep_scale(drop) if keep[i][j] else 0.0


def _head_forward(q, k, v, scale, offset=0, window=0, keep=None, drop=0.0):
    D = len(q[0])
    o = []
    lse = []
    for i in range(len(q)):
        keys = _keys(i, len(k), offset, window)
        if not keys:
            o.append([0.0] * D)
            lse.append(-math.inf)
            continue
        s = []
        for j in keys:
            acc = 0.0
            for d in range(D):
                acc += q[i][d] * k[j][d]
            s.append(scale * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = 0.0
        for x in w:
            z += x
        row = []
        for d in range(D):
            acc = 0.0
            for n, j in enumerate(keys):
                acc += w[n] * _factor(keep, i, j, drop) * v[j][d]
            row.append(acc / z)
        o.append(row)
        lse.append(m + math.log(z))
    return o, lse


def _head_backward(q, k, v, do, scale, offset=0, window=0, keep=None, drop=0.0):
    D = len(q[0])
    dq = [[0.0] * D for _ in range(len(q))]
    dk = [[0.0] * D for _ in range(len(k))]
    dv = [[0.0] * D for _ in range(len(k))]
    for i in range(len(q)):
        keys = _keys(i, len(k), offset, window)
        if not keys:
            continue
        s = []
        for j in keys:
            acc = 0.0
            for d in range(D):
                acc += q[i][d] * k[j][d]
            s.append(scale * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = 0.0
        for x in w:
            z += x
        p = [x / z for x in w]
        # o_i = sum_j p_ij f_ij v_j (f: dropout factor, 1 without dropout), so
        # dL/dp_ij = f_ij (do_i . v_j) and dL/dv_j += p_ij f_ij do_i
        g = []
        for n, j in enumerate(keys):
            f = _factor(keep, i, j, drop)
            acc = 0.0
            for d in range(D):
                acc += do[i][d] * v[j][d]
                dv[j][d] += p[n] * f * do[i][d]
            g.append(f * acc)
        # softmax: dL/ds_ij = p_ij (g_ij - sum_k p_ik g_ik)
        mean = 0.0
        for n in range(len(keys)):
            mean += p[n] * g[n]
        for n, j in enumerate(keys):
            ds = p[n] * (g[n] - mean)
            # s_ij = scale * q_i . k_j
            for d in range(D):
                dq[i][d] += scale * ds * k[j][d]
                dk[j][d] += scale * ds * q[i][d]
    return dq, dk, dv


def _kh(keep, b, h):
    return None if keep is None else keep[b][h]


def forward(q, k, v, scale, offset=0, window=0, keep=None, drop=0.0):
    """Returns ``(o, lse)`` as nested lists."""
    o, lse = [], []
    for b in range(len(q)):
        ob, lb = [], []
        for h in range(len(q[b])):
            oh, lh = _head_forward(q[b][h], k[b][h], v[b][h], scale, offset, window,
                                   _kh(keep, b, h), drop)
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse


def backward(q, k, v, do, scale, offset=0, window=0, keep=None, drop=0.0):
    """Returns ``(dq, dk, dv)`` as nested lists for L = sum(O * dO)."""
    dq, dk, dv = [], [], []
    for b in range(len(q)):
        qb, kb, vb = [], [], []
        for h in range(len(q[b])):
            a, c, e = _head_backward(q[b][h], k[b][h], v[b][h], do[b][h], scale, offset, window,
                                     _kh(keep, b, h), drop)
            qb.append(a)
            kb.append(c)
            vb.append(e)
        dq.append(qb)
        dk.append(kb)
        dv.append(vb)
    return dq, dk, dv
