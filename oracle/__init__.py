"""Plain, slow CPU oracle for batched multi-head causal self-attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers or constants) and imports
nothing from the product package.

Two independent formulations live here:

* :mod:`oracle.attention` -- the definition written out in float64 numpy with
  an explicit T x T score matrix, an explicit mask, a row softmax and plain
  matrix products; the backward pass is the chain rule through those steps.
* :mod:`oracle.bruteforce` -- the same definition as pure-Python scalar loops
  (no numpy at all), used on tiny shapes to pin the vectorised oracle.

What the oracle computes (pages: "Let's build GPT: from scratch, in code,
spelled out", lecture chapters "version 3: adding softmax", "THE CRUX OF THE
VIDEO: version 4: self-attention", note 6 on "scaled" self-attention and the
two listed corrections; nanoGPT README; minGPT README)::

    S     = scale * Q K^T                 (per batch element and head)
    S_ij  = -inf  where j > i             (future keys are invisible)
    P     = row softmax of S              (over keys)
    O     = P V
    lse_i = log sum_j exp(S_ij)           (natural log, kept for backward)

Every function here is pinned by ``tests/test_oracle.py`` against facts that
do not come from this code (brute-force loops, the lecture's prefix-mean
special case computed two other ways, hand-derived closed forms, invariants,
finite differences and the float64 SDPA routine of the PyTorch CPU build).
No function is "parity unpinned".
"""

from . import attention, bruteforce  # noqa: F401
