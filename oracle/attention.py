"""float64 definition of causal scaled dot-product self-attention (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Not on the product
path; imports nothing from the product package.

The steps follow the "Let's build GPT: from scratch, in code, spelled out"
lecture description page in its own order:

* chapter "the trick in self-attention: matrix multiply as weighted
  aggregation" and "version 4: self-attention": every position emits a query,
  a key and a value, affinities are query-key dot products, and the output is
  the affinity-weighted sum of values;
* chapter "version 3: adding softmax": the weights are a row softmax of the
  masked affinities;
* correction at 00:57:00: tokens from the *future* cannot communicate, so a
  query at position i sees keys j <= i (its own position included, as in the
  "version 1: averaging past context" chapter);
* note 6 and the correction at 01:20:05: affinities are scaled by
  1/sqrt(head_size); the scale is an explicit argument here;
* chapter "multi-headed self-attention", exercise EX1 and the chapter
  "batched multi-headed self-attention": heads are one more batch dimension,
  and note 3 says batch elements never communicate.

Layout: every tensor is ``[B, H, T, D]`` (``lse`` is ``[B, H, T]``).  Inputs
of any float dtype are upcast exactly to float64; ``scale`` is taken as the
float32 value the GPU receives, widened to float64.

The backward pass is the chain rule through the same explicit steps for the
scalar loss L = sum(O * dO), so dL/dO = dO:

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)        (softmax Jacobian)
    dQ = scale * dS K
    dK = scale * dS^T Q
"""

import numpy as np


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _scale64(scale):
    # The library receives a float32 scale; the oracle uses that same value.
    return float(np.float32(scale))


def _heads(B, H, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [tuple(bh) for bh in heads]


def scores(q, k, scale):
    """Masked, scaled score matrix S for one (batch, head): ``[T, T]``.

    Entries above the diagonal (keys in the future of the query) are -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    T = q.shape[0]
    s = _scale64(scale) * (q @ k.T)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s[future] = -np.inf
    return s


def probabilities(q, k, scale):
    """Row softmax of the masked scores for one (batch, head): ``[T, T]``."""
    s = scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def forward_head(q, k, v, scale):
    """One (batch, head): returns ``(O [T, D], lse [T])`` in float64."""
    s = scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ _as_f64(v)
    lse = (m + np.log(l))[:, 0]
    return o, lse


def backward_head(q, k, v, do, scale):
    """One (batch, head): returns ``(dQ, dK, dV)``, each ``[T, D]`` float64."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    sc = _scale64(scale)
    p = probabilities(q, k, scale)
    dv = p.T @ do
    dp = do @ v.T
    row = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - row)
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def forward(q, k, v, scale, heads=None):
    """Batched forward over ``[B, H, T, D]`` inputs.

    ``heads`` optionally lists the (b, h) pairs to compute; the others are
    left as NaN so that a caller cannot mistake them for results.
    Returns ``(O [B,H,T,D], lse [B,H,T])`` in float64.
    """
    q = np.asarray(q)
    B, H, T, D = q.shape
    o = np.full((B, H, T, D), np.nan)
    lse = np.full((B, H, T), np.nan)
    for b, h in _heads(B, H, heads):
        o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale)
    return o, lse


def backward(q, k, v, do, scale, heads=None):
    """Batched backward; returns ``(dQ, dK, dV)`` as ``[B,H,T,D]`` float64.

    Heads not listed in ``heads`` are NaN.
    """
    q = np.asarray(q)
    B, H, T, D = q.shape
    dq = np.full((B, H, T, D), np.nan)
    dk = np.full((B, H, T, D), np.nan)
    dv = np.full((B, H, T, D), np.nan)
    for b, h in _heads(B, H, heads):
        dq[b, h], dk[b, h], dv[b, h] = backward_head(
            q[b, h], k[b, h], v[b, h], do[b, h], scale)
    return dq, dk, dv
