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
* correction at 00:57:00: a query never looks at later positions, so a
  query at position i sees keys j <= i (its own position included, as in the
  "version 1: averaging past context" chapter);
* note 6 and the correction at 01:20:05: affinities are scaled by
  1/sqrt(head_size); the scale is an explicit argument here;
* chapter "multi-headed self-attention", exercise EX1 and the chapter
  "batched multi-headed self-attention": heads are one more batch dimension,
  and note 3 says batch elements never communicate;
* chapter "scaling up the model! ... adding dropout" (with the nanoGPT
  README's `--dropout` flag): optional dropout on the attention weights.
  Read as: the softmax weights P are multiplied by a keep mask M and by the
  keep scale s = 2^16 / (2^16 - thr) (the inverse of the keep probability
  the generator's 16-bit threshold thr = ceil(p * 2^16) realises, so the
  dropped-out weights are unbiased) before they weight the values; lse is
  the normaliser of the softmax itself, before dropout.  M comes from
  oracle.philox.keep_mask, s from oracle.philox.keep_scale.

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

With dropout, Pd = P * M * s replaces P in O = Pd V and dV = Pd^T dO,
and dP = (dO V^T) * M * s enters the softmax Jacobian.
"""

import numpy as np

from oracle import philox


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _scale64(scale):
    # The library receives a float32 scale; the oracle uses that same value.
    return float(np.float32(scale))


def _heads(B, H, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [tuple(bh) for bh in heads]


def visible(Tq, Tk, offset=0, window=0):
    """Boolean ``[Tq, Tk]`` matrix of the (query, key) pairs that attend.

    Query i sees key j when j <= i + offset (nothing from its future); with
    window > 0 it also needs j > i + offset - window (a local band of the
    `window` most recent positions, the "locally banded" layers of GPT-3 in
    the minGPT README notes).  offset = Tk - Tq lines the last query up with
    the last key (new tokens appended to a context).  offset = 0, window = 0,
    Tq = Tk is the plain causal mask.
    """
    i = np.arange(Tq)[:, None] + offset
    j = np.arange(Tk)[None, :]
    ok = j <= i
    if window > 0:
        ok &= j > i - window
    return ok


def scores(q, k, scale, offset=0, window=0):
    """Masked, scaled score matrix S for one (batch, head): ``[Tq, Tk]``.

    Entries of keys a query may not see are -inf (for plain causal
    attention: everything above the diagonal).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    s = _scale64(scale) * (q @ k.T)
    s[~visible(q.shape[0], k.shape[0], offset, window)] = -np.inf
    return s


def _softmax_rows(s):
    """Row softmax; a row with no visible key gets all-zero weights."""
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m[empty] = 0.0
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
    lse = np.where(empty, -np.inf, (m + np.log(np.where(l > 0, l, 1.0)))[:, 0])
    return p, lse


def probabilities(q, k, scale, offset=0, window=0):
    """Row softmax of the masked scores for one (batch, head)."""
    return _softmax_rows(scores(q, k, scale, offset, window))[0]


def _drop_factor(keep, p):
    """Per-weight dropout factor M * s (None without dropout), s the keep
    scale of oracle.philox.keep_scale: the inverse of the keep probability
    the generator's threshold realises."""
    if keep is None:
        return None
    return keep.astype(np.float64) * philox.keep_scale(p)


def forward_head(q, k, v, scale, offset=0, window=0, keep=None, p=0.0):
    """One (batch, head): returns ``(O [Tq, D], lse [Tq])`` in float64.

    A query row that sees no key (possible only with a negative offset) has
    O = 0 and lse = -inf.  ``keep`` ([Tq, Tk] booleans) applies dropout with
    probability ``p`` to the weights.
    """
    w, lse = _softmax_rows(scores(q, k, scale, offset, window))
    f = _drop_factor(keep, p)
    if f is not None:
        w = w * f
    o = w @ _as_f64(v)
    return o, lse


def backward_head(q, k, v, do, scale, offset=0, window=0, keep=None, p=0.0):
    """One (batch, head): returns ``(dQ [Tq, D], dK [Tk, D], dV [Tk, D])``."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    sc = _scale64(scale)
    w = probabilities(q, k, scale, offset, window)
    f = _drop_factor(keep, p)
    wd = w if f is None else w * f
    dv = wd.T @ do
    dp = do @ v.T
    if f is not None:
        dp = dp * f
    row = (w * dp).sum(axis=1, keepdims=True)
    ds = w * (dp - row)
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def _keep(b, h, H, Tq, Tk, dropout, seed, stream):
    if dropout <= 0:
        return None
    return philox.keep_mask(b * H + h, Tq, Tk, dropout, seed, stream)


def forward(q, k, v, scale, heads=None, offset=0, window=0, dropout=0.0, seed=0, stream=0):
    """Batched forward over ``[B, H, Tq, D]`` queries and ``[B, H, Tk, D]``
    keys/values.

    ``heads`` optionally lists the (b, h) pairs to compute; the others are
    left as NaN so that a caller cannot mistake them for results.
    ``dropout``/``seed``/``stream`` select the keep mask of each head
    (oracle.philox.keep_mask with n = b * H + h).
    Returns ``(O [B,H,Tq,D], lse [B,H,Tq])`` in float64.
    """
    q = np.asarray(q)
    B, H, Tq, D = q.shape
    Tk = np.asarray(k).shape[2]
    o = np.full((B, H, Tq, D), np.nan)
    lse = np.full((B, H, Tq), np.nan)
    for b, h in _heads(B, H, heads):
        keep = _keep(b, h, H, Tq, Tk, dropout, seed, stream)
        o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale, offset, window,
                                          keep, dropout)
    return o, lse


def backward(q, k, v, do, scale, heads=None, offset=0, window=0, dropout=0.0, seed=0,
             stream=0):
    """Batched backward; returns ``(dQ, dK, dV)`` in float64 (dQ like q,
    dK and dV like k).  Heads not listed in ``heads`` are NaN.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    dq = np.full((B, H, Tq, D), np.nan)
    dk = np.full((B, H, Tk, D), np.nan)
    dv = np.full((B, H, Tk, D), np.nan)
    for b, h in _heads(B, H, heads):
        keep = _keep(b, h, H, Tq, Tk, dropout, seed, stream)
        dq[b, h], dk[b, h], dv[b, h] = backward_head(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, offset, window, keep, dropout)
    return dq, dk, dv
