"""Causal scaled dot-product self-attention for AMD MI355X (gfx950).

Thin Python binding over ``libgptattn.so`` (C ABI declared in
``include/gptattn.h``).  This module only marshals arguments: it checks
tensor shapes/dtypes/devices, allocates output tensors with PyTorch (device
memory is PyTorch's job here) and passes raw device pointers plus the current
HIP stream.  Every arithmetic step runs in the library's HIP kernels; there
is no fallback.  If the library is missing, every call raises.

Operation (lecture description "Let's build GPT: from scratch, in code,
spelled out": "version 3: adding softmax", "version 4: self-attention",
note 6 and the corrections at 00:57:00 and 01:20:05; heads as a batch
dimension per EX1):

    O   = softmax(scale * Q K^T, keys j <= i only) V
    lse = log sum_{j <= i} exp(scale * q_i . k_j)

Tensors are ``[B, H, T, D]`` contiguous, bfloat16 (D in {64, 128}) or
float32 (D in {16, 32, 64}); ``lse`` is ``[B, H, T]`` float32.

The ``*_ex`` calls take any ``[B, H, T, D]`` view whose last dimension is
contiguous (for example q, k and v sliced out of one packed ``[B, T, 3C]``
projection output, see :func:`split_qkv`), allow ``Tq != Tk`` and take the
two mask parameters of ``gptattn_problem``: query i sees key j when
``j <= i + causal_offset`` and, with ``window > 0``, ``j > i + causal_offset
- window``.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "fwd", "bwd", "bwd_noalloc", "bwd_dq", "bwd_dkdv", "fwd_ex", "bwd_ex", "split_qkv", "attention",
    "GPTAttnFunction", "workspace_bytes", "ex_workspace_bytes", "status_string", "version",
    "library", "LIB_PATH", "Tensor", "Problem", "DTYPE_BF16", "DTYPE_F32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptattn.so")

_LIB = None
_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

DTYPE_BF16 = 0
DTYPE_F32 = 1


class Tensor(ctypes.Structure):
    """``gptattn_tensor``: element (b, h, t, d) at data + b*stride_b +
    h*stride_h + t*stride_t + d (elements)."""
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_longlong),
                ("stride_h", ctypes.c_longlong), ("stride_t", ctypes.c_longlong)]


class Problem(ctypes.Structure):
    """``gptattn_problem``."""
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("Tq", ctypes.c_int),
                ("Tk", ctypes.c_int), ("D", ctypes.c_int), ("causal_offset", ctypes.c_int),
                ("window", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("dropout", ctypes.c_float), ("rng_stream", ctypes.c_uint),
                ("seed", ctypes.c_ulonglong)]


_tp = ctypes.POINTER(Tensor)
_pp = ctypes.POINTER(Problem)

# name -> (restype, argtypes); mirrors include/gptattn.h
SIGNATURES = {
    "gptattn_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p]),
    "gptattn_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "gptattn_bwd_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p]),
    "gptattn_bwd_dq": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "gptattn_bwd_dkdv": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "gptattn_fwd_f32": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p]),
    "gptattn_bwd_dq_f32": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "gptattn_bwd_dkdv_f32": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz,
                                  _p]),
    "gptattn_bwd_f32": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "gptattn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "gptattn_fwd_ex": (_i, [_pp, _tp, _tp, _tp, _tp, _p, _p]),
    "gptattn_bwd_ex": (_i, [_pp, _tp, _tp, _tp, _tp, _tp, _p, _tp, _tp, _tp, _p, _sz, _p]),
    "gptattn_bwd_ex_workspace_bytes": (_sz, [_pp]),
    "gptattn_status_string": (ctypes.c_char_p, [_i]),
    "gptattn_version": (_i, []),
}


def library():
    """Load ``libgptattn.so`` (once) and return the ctypes handle."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgptattn.so is not built (expected at %s); build it with "
                "`python -m causal_self_attention_gptattn_amd._build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def status_string(rc):
    return library().gptattn_status_string(int(rc)).decode()


def version():
    return library().gptattn_version()


def workspace_bytes(B, H, T, D, is_f32=False):
    return library().gptattn_bwd_workspace_bytes(B, H, T, D, 1 if is_f32 else 0)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed: %s" % (what, status_string(rc)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _validate(ref, *others):
    if ref.dim() != 4:
        raise ValueError("expected [B, H, T, D] tensors, got shape %s" % (tuple(ref.shape),))
    if not ref.is_cuda:
        raise ValueError("tensors must live on a GPU")
    if ref.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32, got %s" % ref.dtype)
    for t in (ref,) + others:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and o, dO) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, T, D]")


def _scale(scale, D):
    return float(1.0 / math.sqrt(D)) if scale is None else float(scale)


def fwd(q, k, v, scale=None, out=None, lse=None):
    """Forward pass; returns ``(o, lse)``.

    ``out``/``lse`` may be passed to reuse buffers (they are overwritten).
    """
    _validate(q, k, v)
    B, H, T, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    _validate(q, out)
    if lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    lib = library()
    fn = lib.gptattn_fwd if q.dtype == torch.bfloat16 else lib.gptattn_fwd_f32
    with torch.cuda.device(q.device):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, T, D,
                _scale(scale, D), _stream(q.device))
    _check(rc, "gptattn_fwd")
    return out, lse


def bwd(q, k, v, o, do, lse, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass for dL/dO = ``do``; returns ``(dq, dk, dv)``."""
    _validate(q, k, v, o, do)
    B, H, T, D = q.shape
    if lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _validate(q, dq, dk, dv)
    is_f32 = q.dtype == torch.float32
    need = workspace_bytes(B, H, T, D, is_f32)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    lib = library()
    fn = lib.gptattn_bwd_f32 if is_f32 else lib.gptattn_bwd
    with torch.cuda.device(q.device):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                _ptr(dv), B, H, T, D, _scale(scale, D), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(rc, "gptattn_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, scale=None, dq=None, dk=None, dv=None):
    """Backward pass (bfloat16) through ``gptattn_bwd_noalloc``: no
    workspace; the library's fixed scratch array takes its place (at most
    ``NOALLOC_MAX_ROWS`` = B*H*T rows; overlapping calls on one GPU race)."""
    _validate(q, k, v, o, do)
    B, H, T, D = q.shape
    if lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _validate(q, dq, dk, dv)
    with torch.cuda.device(q.device):
        rc = library().gptattn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                           _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, T, D,
                                           _scale(scale, D), _stream(q.device))
    _check(rc, "gptattn_bwd_noalloc")
    return dq, dk, dv


NOALLOC_MAX_ROWS = 1 << 20


def _rows_ok(t, q):
    B, H, T, _ = q.shape
    if t.shape != (B, H, T) or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")


def _ws(workspace, q):
    B, H, T, D = q.shape
    need = workspace_bytes(B, H, T, D, q.dtype == torch.float32)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def bwd_dq(q, k, v, o, do, lse, scale=None, dq=None, workspace=None):
    """First backward launch: dq, plus the row term stored in ``workspace``.

    Returns ``(dq, workspace)``; pass that workspace to :func:`bwd_dkdv`.
    """
    _validate(q, k, v, o, do)
    _rows_ok(lse, q)
    B, H, T, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    _validate(q, dq)
    workspace, nbytes = _ws(workspace, q)
    lib = library()
    fn = lib.gptattn_bwd_dq_f32 if q.dtype == torch.float32 else lib.gptattn_bwd_dq
    with torch.cuda.device(q.device):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), B, H, T, D,
                _scale(scale, D), _ptr(workspace), nbytes, _stream(q.device))
    _check(rc, "gptattn_bwd_dq")
    return dq, workspace


def bwd_dkdv(q, k, v, do, lse, workspace, scale=None, dk=None, dv=None):
    """Second backward launch: dk, dv from the row term in ``workspace``."""
    _validate(q, k, v, do)
    _rows_ok(lse, q)
    B, H, T, D = q.shape
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _validate(q, dk, dv)
    lib = library()
    fn = lib.gptattn_bwd_dkdv_f32 if q.dtype == torch.float32 else lib.gptattn_bwd_dkdv
    with torch.cuda.device(q.device):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dk), _ptr(dv), B, H, T, D,
                _scale(scale, D), _ptr(workspace), workspace.numel() * workspace.element_size(),
                _stream(q.device))
    _check(rc, "gptattn_bwd_dkdv")
    return dk, dv


# ---------------------------------------------------------------------------
# Strided views, Tq != Tk, shifted and banded masks (gptattn_*_ex)
# ---------------------------------------------------------------------------

def split_qkv(x, n_head):
    """Views q, k, v ``[B, H, T, D]`` of a packed ``[B, T, 3C]`` projection
    output (q, k, v concatenated along the last axis, each C = H*D wide,
    heads in order), without copying."""
    B, T, C3 = x.shape
    C = C3 // 3
    xv = x.view(B, T, 3, n_head, C // n_head)
    return tuple(xv[:, :, i].transpose(1, 2) for i in range(3))


def _tensor(t):
    if t.stride(3) != 1:
        raise ValueError("the last (head) dimension must be contiguous")
    st = [0 if t.shape[i] == 1 else t.stride(i) for i in range(3)]
    return Tensor(t.data_ptr(), st[0], st[1], st[2])


def _view_ok(t):
    """Whether the strided calls take ``t`` as it is: 16-byte aligned data,
    a contiguous last dimension, non-negative strides that are whole 16-byte
    units, rows that do not overlap (row stride >= D unless there is a
    single row) and row strides of at most 2^23 elements.  Autograd can hand
    the backward pass a gradient that fails this (``o.sum(dim=2)`` gives
    dO a row stride of 0); such a tensor is copied first."""
    unit = 16 // t.element_size()
    st = [0 if t.shape[i] == 1 else t.stride(i) for i in range(3)]
    return (t.data_ptr() % 16 == 0 and t.stride(3) == 1 and all(s >= 0 for s in st)
            and all(s % unit == 0 for s in st)
            and (t.shape[2] == 1 or t.stride(2) >= t.shape[3]) and st[2] <= (1 << 23))


def _problem(q, k, scale, causal_offset, window, dropout=0.0, seed=0, rng_stream=0):
    B, H, Tq, D = q.shape
    dt = DTYPE_F32 if q.dtype == torch.float32 else DTYPE_BF16
    return Problem(B, H, Tq, k.shape[2], D, int(causal_offset), int(window),
                   _scale(scale, D), dt, float(dropout), int(rng_stream) & 0xFFFFFFFF,
                   int(seed) & 0xFFFFFFFFFFFFFFFF)


def _validate_ex(q, k, v, *rows_q):
    for t in (q, k, v) + rows_q:
        if t.dim() != 4:
            raise ValueError("expected [B, H, T, D] tensors, got shape %s" % (tuple(t.shape),))
        if not t.is_cuda or t.device != q.device:
            raise ValueError("tensors must live on the same GPU")
        if t.dtype != q.dtype or q.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("tensors must all be bfloat16 or all float32")
    B, H, Tq, D = q.shape
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != D:
        raise ValueError("k and v must be [B, H, Tk, D] with q's B, H and D")
    for t in rows_q:
        if t.shape != q.shape:
            raise ValueError("o, dO and dq must have q's shape")


def ex_workspace_bytes(q, k, scale=None, causal_offset=0, window=0):
    pb = _problem(q, k, scale, causal_offset, window)
    return library().gptattn_bwd_ex_workspace_bytes(ctypes.byref(pb))


def fwd_ex(q, k, v, scale=None, causal_offset=0, window=0, out=None, lse=None, dropout=0.0,
           seed=0, rng_stream=0):
    """Forward pass over strided ``[B, H, T, D]`` views; returns ``(o, lse)``.

    ``out`` may be any view of q's shape with a contiguous last dimension
    (for example a ``[B, T, H, D]`` buffer transposed to ``[B, H, T, D]``).
    ``dropout`` > 0 drops attention weights; the mask is a function of
    (``seed``, ``rng_stream``, head, query, key), so the backward call must
    get the same three values.
    """
    _validate_ex(q, k, v)
    B, H, Tq, D = q.shape
    out = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _validate_ex(q, k, v, out)
    _rows_ok(lse, q)
    pb = _problem(q, k, scale, causal_offset, window, dropout, seed, rng_stream)
    ts = [_tensor(t) for t in (q, k, v, out)]
    with torch.cuda.device(q.device):
        rc = library().gptattn_fwd_ex(ctypes.byref(pb), *[ctypes.byref(t) for t in ts],
                                      _ptr(lse), _stream(q.device))
    _check(rc, "gptattn_fwd_ex")
    return out, lse


def bwd_ex(q, k, v, o, do, lse, scale=None, causal_offset=0, window=0, dq=None, dk=None,
           dv=None, workspace=None, dropout=0.0, seed=0, rng_stream=0):
    """Backward pass over strided views; returns ``(dq, dk, dv)``.  The
    gradients may be views into one packed buffer (see :func:`split_qkv`)."""
    _validate_ex(q, k, v, o, do)
    _rows_ok(lse, q)
    fresh = dict(memory_format=torch.contiguous_format)
    dq = torch.empty_like(q, **fresh) if dq is None else dq
    dk = torch.empty_like(k, **fresh) if dk is None else dk
    dv = torch.empty_like(v, **fresh) if dv is None else dv
    _validate_ex(q, dk, dv, dq)
    pb = _problem(q, k, scale, causal_offset, window, dropout, seed, rng_stream)
    lib = library()
    need = lib.gptattn_bwd_ex_workspace_bytes(ctypes.byref(pb))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ts = [_tensor(t) for t in (q, k, v, o, do)]
    gs = [_tensor(t) for t in (dq, dk, dv)]
    with torch.cuda.device(q.device):
        rc = lib.gptattn_bwd_ex(ctypes.byref(pb), *[ctypes.byref(t) for t in ts], _ptr(lse),
                                *[ctypes.byref(t) for t in gs], _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(rc, "gptattn_bwd_ex")
    return dq, dk, dv


class GPTAttnFunction(torch.autograd.Function):
    """Autograd wrapper: saves (q, k, v, o, lse) and calls the backward
    launches.  Inputs may be strided views (for example from
    :func:`split_qkv`)."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, causal_offset=0, window=0, dropout=0.0, seed=0,
                rng_stream=0):
        o, lse = fwd_ex(q, k, v, scale, causal_offset, window, dropout=dropout, seed=seed,
                        rng_stream=rng_stream)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (scale, causal_offset, window)
        ctx.drop = dict(dropout=dropout, seed=seed, rng_stream=rng_stream)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if not _view_ok(do):
            do = do.contiguous()
        dq, dk, dv = bwd_ex(q, k, v, o, do, lse, *ctx.args, **ctx.drop)
        return dq, dk, dv, None, None, None, None, None, None


def attention(q, k, v, scale=None, causal_offset=0, window=0, dropout=0.0, seed=0,
              rng_stream=0):
    """Differentiable causal self-attention over ``[B, H, T, D]`` views
    (``Tq`` queries, ``Tk`` keys; mask and dropout parameters as in
    :func:`fwd_ex`)."""
    return GPTAttnFunction.apply(q, k, v, scale, causal_offset, window, dropout, seed,
                                 rng_stream)
