"""C-ABI checks of the strided entry points (gptattn_fwd_ex / gptattn_bwd_ex)
that need no GPU: every call here is refused by validation before any HIP
call.  Layouts the overlap test accepts are recognised by the status that
comes after it: gptattn_bwd_ex checks the views first and the workspace size
last, so an accepted layout with a too-small workspace returns WORKSPACE."""

import ctypes

import pytest

import causal_self_attention_gptattn_amd as G

SUCCESS, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH = 0, 1, 2, 3, 4
BASE = [0x100000000 * (i + 1) for i in range(16)]  # fake, aligned, far apart


@pytest.fixture(scope="module")
def lib():
    return G.library()


def prob(B=2, H=2, Tq=8, Tk=8, D=64, off=0, win=0, scale=0.125, dtype=G.DTYPE_BF16,
         dropout=0.0):
    return G.Problem(B, H, Tq, Tk, D, off, win, scale, dtype, dropout, 0, 0)


def dense(base, p, rows):
    return G.Tensor(base, p.H * rows * p.D, rows * p.D, p.D)


def packed(base, p, which, elem=2):
    """q/k/v slot `which` of a packed [B][T][3][H][D] buffer at `base`."""
    C = p.H * p.D
    return G.Tensor(base + which * C * elem, p.Tq * 3 * C, p.D, 3 * C)


def fwd_ex(lib, p, q, k, v, o, lse=BASE[9]):
    return lib.gptattn_fwd_ex(ctypes.byref(p) if p is not None else None, *(
        ctypes.byref(t) if t is not None else None for t in (q, k, v, o)),
        ctypes.c_void_p(lse), None)


def bwd_ex(lib, p, ins, outs, lse=BASE[9], ws=BASE[10], ws_bytes=1):
    return lib.gptattn_bwd_ex(
        ctypes.byref(p), *(ctypes.byref(t) for t in ins), ctypes.c_void_p(lse),
        *(ctypes.byref(t) for t in outs), ctypes.c_void_p(ws), ws_bytes, None)


def dense_ins(p):
    return [dense(BASE[0], p, p.Tq), dense(BASE[1], p, p.Tk), dense(BASE[2], p, p.Tk),
            dense(BASE[3], p, p.Tq), dense(BASE[4], p, p.Tq)]


def dense_outs(p):
    return [dense(BASE[5], p, p.Tq), dense(BASE[6], p, p.Tk), dense(BASE[7], p, p.Tk)]


def test_workspace_bytes_ex(lib):
    p = prob(B=3, H=5, Tq=7, Tk=40)
    assert lib.gptattn_bwd_ex_workspace_bytes(ctypes.byref(p)) == 2 * 3 * 5 * 7 * 4
    assert lib.gptattn_bwd_ex_workspace_bytes(None) == 0
    assert lib.gptattn_bwd_ex_workspace_bytes(ctypes.byref(prob(Tq=0))) == 0


def test_dense_layout_is_accepted(lib):
    p = prob()
    assert bwd_ex(lib, p, dense_ins(p), dense_outs(p)) == WORKSPACE


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(H=0), dict(Tq=0), dict(Tk=0), dict(D=0), dict(win=-1),
    dict(off=2 ** 29 + 1), dict(off=-2 ** 29 - 1), dict(Tq=2 ** 29 + 1), dict(win=2 ** 29 + 1),
    dict(scale=0.0), dict(scale=float("nan")), dict(dtype=2), dict(dtype=-1),
    dict(B=2 ** 20, H=2 ** 10, Tq=2 ** 12, Tk=2 ** 12),
    dict(dropout=-0.1), dict(dropout=1.0), dict(dropout=float("nan")), dict(dropout=float("inf")),
])
def test_bad_problem(lib, kw):
    p = prob(**kw)
    ins = dense_ins(p)
    assert fwd_ex(lib, p, *ins[:3], dense(BASE[5], p, max(p.Tq, 1))) == INVALID
    assert bwd_ex(lib, p, ins, dense_outs(p)) == INVALID


def test_null_problem(lib):
    p = prob()
    assert fwd_ex(lib, None, *dense_ins(p)[:3], dense(BASE[5], p, p.Tq)) == INVALID


@pytest.mark.parametrize("D,dtype", [(32, G.DTYPE_BF16), (96, G.DTYPE_BF16),
                                     (128, G.DTYPE_F32), (8, G.DTYPE_F32)])
def test_unsupported_head(lib, D, dtype):
    p = prob(D=D, dtype=dtype)
    assert fwd_ex(lib, p, *dense_ins(p)[:3], dense(BASE[5], p, p.Tq)) == UNSUPPORTED


@pytest.mark.parametrize("field,value", [
    ("data", 0), ("data", BASE[0] + 8), ("stride_t", 60), ("stride_h", -64), ("stride_b", 12),
    ("stride_t", 2 ** 23 + 8), ("stride_t", 56), ("stride_t", 0),
])
def test_bad_tensor(lib, field, value):
    p = prob()
    ins = dense_ins(p)
    setattr(ins[1], field, value)
    assert fwd_ex(lib, p, *ins[:3], dense(BASE[5], p, p.Tq)) == INVALID
    assert bwd_ex(lib, p, ins, dense_outs(p)) == INVALID


def test_f32_stride_granule(lib):
    p = prob(D=16, dtype=G.DTYPE_F32)
    ins = dense_ins(p)
    ins[0].stride_t = 20           # 80 bytes: a multiple of 16
    assert bwd_ex(lib, p, ins, dense_outs(p)) == WORKSPACE
    ins[0].stride_t = 18           # 72 bytes: not
    assert bwd_ex(lib, p, ins, dense_outs(p)) == INVALID


def test_packed_inputs_and_gradients_are_accepted(lib):
    """q, k, v read from one packed projection output and dq, dk, dv written
    into one packed gradient buffer interleave but do not overlap."""
    p = prob(B=2, H=3, Tq=16, Tk=16, D=64)
    ins = [packed(BASE[0], p, 0), packed(BASE[0], p, 1), packed(BASE[0], p, 2),
           dense(BASE[3], p, p.Tq), dense(BASE[4], p, p.Tq)]
    outs = [packed(BASE[5], p, 0), packed(BASE[5], p, 1), packed(BASE[5], p, 2)]
    assert bwd_ex(lib, p, ins, outs) == WORKSPACE
    # dq written as a [B][T][H][D] buffer (one contiguous run per batch entry)
    outs = dense_outs(p)
    outs[0] = G.Tensor(BASE[5], p.Tq * p.H * p.D, p.D, p.H * p.D)
    assert bwd_ex(lib, p, ins, outs) == WORKSPACE


@pytest.mark.parametrize("case", ["same_slot", "half_slot", "over_input", "into_lse"])
def test_packed_overlaps_are_refused(lib, case):
    p = prob(B=2, H=3, Tq=16, Tk=16, D=64)
    C2 = p.H * p.D * 2
    ins = [packed(BASE[0], p, 0), packed(BASE[0], p, 1), packed(BASE[0], p, 2),
           dense(BASE[3], p, p.Tq), dense(BASE[4], p, p.Tq)]
    outs = [packed(BASE[5], p, 0), packed(BASE[5], p, 1), packed(BASE[5], p, 2)]
    lse = BASE[9]
    if case == "same_slot":
        outs[1] = packed(BASE[5], p, 0)
    elif case == "half_slot":
        outs[1].data = outs[0].data + C2 // 2
    elif case == "over_input":
        outs[0] = packed(BASE[0], p, 2)     # dq on top of v
    elif case == "into_lse":
        lse = BASE[5] + C2                  # lse inside the packed gradient buffer
    assert bwd_ex(lib, p, ins, outs, lse=lse) == INVALID


def test_output_must_not_repeat_elements(lib):
    p = prob()
    outs = dense_outs(p)
    outs[0].stride_h = 0                     # every head written to the same rows
    assert bwd_ex(lib, p, dense_ins(p), outs) == INVALID
    outs = dense_outs(p)
    outs[2].stride_t = 32                    # rows of 64 elements, 32 apart
    assert bwd_ex(lib, p, dense_ins(p), outs) == INVALID


def test_broadcast_inputs_are_accepted(lib):
    """One set of keys and values for all heads (stride_h = 0) is a valid input."""
    p = prob(H=4)
    ins = dense_ins(p)
    ins[1].stride_h = 0
    ins[2].stride_h = 0
    assert bwd_ex(lib, p, ins, dense_outs(p)) == WORKSPACE


def test_workspace_overlapping_output_is_refused(lib):
    p = prob()
    assert bwd_ex(lib, p, dense_ins(p), dense_outs(p), ws=BASE[6]) == INVALID


def test_tq_tk_shapes(lib):
    """Views are sized by their own lengths: k and v span Tk rows."""
    p = prob(Tq=1, Tk=100, off=99)
    ins = dense_ins(p)
    outs = dense_outs(p)
    assert bwd_ex(lib, p, ins, outs) == WORKSPACE
    # dv starting 50 rows into dk's Tk-row span overlaps it
    outs[2].data = outs[1].data + 64 * 2 * 50
    assert bwd_ex(lib, p, ins, outs) == INVALID


def test_single_row_ignores_its_stride(lib):
    """With Tq = 1 the row stride of q, o, dO and dq is never used (torch
    reports arbitrary strides for size-1 dimensions)."""
    p = prob(Tq=1, Tk=40, off=39)
    ins = dense_ins(p)
    outs = dense_outs(p)
    for t in (ins[0], ins[3], ins[4], outs[0]):
        t.stride_t = 0
    assert bwd_ex(lib, p, ins, outs) == WORKSPACE


def test_dropout_range_is_accepted(lib):
    for p_ in (0.0, 0.1, 0.999):
        p = prob(dropout=p_)
        assert bwd_ex(lib, p, dense_ins(p), dense_outs(p)) == WORKSPACE
