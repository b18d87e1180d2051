"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (so these
calls never reach a kernel launch)."""

import ctypes
import os
import re

import pytest

import causal_self_attention_gptattn_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptattn.h")

SUCCESS, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH, SCRATCH = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(G.LIB_PATH):
        pytest.fail("libgptattn.so is not built; run __graft_entry__.build()")
    return G.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(G.SIGNATURES), (names, sorted(G.SIGNATURES))
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_in_header():
    text = open(HEADER).read()
    for name, val in (("GPTATTN_SUCCESS", 0), ("GPTATTN_ERROR_INVALID_VALUE", 1),
                      ("GPTATTN_ERROR_NOT_SUPPORTED", 2), ("GPTATTN_ERROR_WORKSPACE", 3),
                      ("GPTATTN_ERROR_LAUNCH", 4), ("GPTATTN_ERROR_SCRATCH", 5)):
        assert re.search(r"\b%s\s*=\s*%d\b" % (name, val), text), name


def test_version_and_strings(lib):
    assert G.version() == 10000
    for code in range(-1, 7):
        s = G.status_string(code)
        assert isinstance(s, str) and s
    assert "NOT_SUPPORTED" in G.status_string(UNSUPPORTED)


def test_workspace_bytes(lib):
    assert G.workspace_bytes(12, 12, 1024, 64) == 2 * 12 * 12 * 1024 * 4
    assert G.workspace_bytes(1, 4, 64, 16, True) == 2 * 4 * 64 * 4
    assert G.workspace_bytes(0, 1, 1, 64) == 0
    assert G.workspace_bytes(1, 1, -3, 64) == 0


# Distinct, 16-byte aligned fake device addresses, far apart.  They are never
# dereferenced: every call below fails validation first.
A = [0x10000000 * (i + 1) for i in range(12)]


def fwd(lib, ptrs=None, B=1, H=1, T=8, D=64, scale=0.125, f32=False):
    p = list(A[:5]) if ptrs is None else ptrs
    fn = lib.gptattn_fwd_f32 if f32 else lib.gptattn_fwd
    return fn(*[ctypes.c_void_p(x) for x in p], B, H, T, D, scale, None)


def bwd(lib, ptrs=None, ws=None, ws_bytes=1 << 20, B=1, H=1, T=8, D=64, scale=0.125, f32=False):
    p = list(A[:9]) if ptrs is None else ptrs
    w = A[10] if ws is None else ws
    fn = lib.gptattn_bwd_f32 if f32 else lib.gptattn_bwd
    return fn(*[ctypes.c_void_p(x) for x in p], B, H, T, D, scale, ctypes.c_void_p(w),
              ws_bytes, None)


@pytest.mark.parametrize("f32", [False, True])
def test_null_pointers(lib, f32):
    D = 16 if f32 else 64
    for i in range(5):
        p = list(A[:5])
        p[i] = 0
        assert fwd(lib, p, D=D, f32=f32) == INVALID
    for i in range(9):
        p = list(A[:9])
        p[i] = 0
        assert bwd(lib, p, D=D, f32=f32) == INVALID


@pytest.mark.parametrize("f32", [False, True])
def test_split_backward_validation(lib, f32):
    D = 16 if f32 else 64
    suffix = "_f32" if f32 else ""
    dq = getattr(lib, "gptattn_bwd_dq" + suffix)
    dkdv = getattr(lib, "gptattn_bwd_dkdv" + suffix)
    P = [ctypes.c_void_p(x) for x in A[:7]]
    W_ = ctypes.c_void_p(A[10])
    for i in range(7):
        p = list(P)
        p[i] = ctypes.c_void_p(0)
        assert dq(*p, 1, 1, 8, D, 0.125, W_, 1 << 20, None) == INVALID
        assert dkdv(*p, 1, 1, 8, D, 0.125, W_, 1 << 20, None) == INVALID
    assert dq(*P, 1, 1, 8, D, 0.125, ctypes.c_void_p(0), 1 << 20, None) == WORKSPACE
    assert dkdv(*P, 1, 1, 8, D, 0.125, W_, 4, None) == WORKSPACE
    assert dq(*P, 1, 1, 8, D + 1, 0.125, W_, 1 << 20, None) == UNSUPPORTED
    # dk written over the workspace the call reads
    p = list(P)
    p[5] = W_
    assert dkdv(*p, 1, 1, 8, D, 0.125, W_, 1 << 20, None) == INVALID
    # dq on top of q
    p = list(P)
    p[6] = P[0]
    assert dq(*p, 1, 1, 8, D, 0.125, W_, 1 << 20, None) == INVALID


def test_misaligned(lib):
    for i in range(5):
        p = list(A[:5])
        p[i] += 8
        assert fwd(lib, p) == INVALID
    p = list(A[:9])
    p[7] += 2
    assert bwd(lib, p) == INVALID
    assert bwd(lib, ws=A[10] + 4) == WORKSPACE


@pytest.mark.parametrize("dims", [(0, 1, 8, 64), (1, 0, 8, 64), (1, 1, 0, 64), (1, 1, 8, 0),
                                  (-1, 1, 8, 64), (1, 1, -5, 64)])
def test_bad_sizes(lib, dims):
    B, H, T, D = dims
    assert fwd(lib, B=B, H=H, T=T, D=D) == INVALID
    assert bwd(lib, B=B, H=H, T=T, D=D) == INVALID


def test_overflowing_sizes(lib):
    big = 2 ** 31 - 1
    assert fwd(lib, B=big, H=big, T=big, D=64) == INVALID


@pytest.mark.parametrize("scale", [0.0, -0.125, float("nan"), float("inf"), float("-inf")])
def test_bad_scale(lib, scale):
    assert fwd(lib, scale=scale) == INVALID
    assert bwd(lib, scale=scale) == INVALID


@pytest.mark.parametrize("D,f32", [(16, False), (32, False), (96, False), (256, False),
                                   (128, True), (8, True), (48, True)])
def test_unsupported_head_size(lib, D, f32):
    assert fwd(lib, D=D, f32=f32) == UNSUPPORTED
    assert bwd(lib, D=D, f32=f32) == UNSUPPORTED


def test_workspace_checks(lib):
    assert bwd(lib, ws=0) == WORKSPACE
    assert bwd(lib, ws_bytes=2 * 8 * 4 - 1) == WORKSPACE  # needs 2*B*H*T*4 = 64 bytes


def test_overlapping_outputs(lib):
    # o on top of q
    p = list(A[:5])
    p[3] = p[0]
    assert fwd(lib, p) == INVALID
    # lse inside o
    p = list(A[:5])
    p[4] = p[3] + 64
    assert fwd(lib, p) == INVALID
    # dq == dk
    p = list(A[:9])
    p[7] = p[6]
    assert bwd(lib, p) == INVALID
    # dv overlaps dO
    p = list(A[:9])
    p[8] = p[4] + 16
    assert bwd(lib, p) == INVALID
    # workspace overlaps lse
    assert bwd(lib, ws=A[5]) == INVALID


def bwd_noalloc(lib, ptrs=None, B=1, H=1, T=8, D=64, scale=0.125):
    p = list(A[:9]) if ptrs is None else ptrs
    return lib.gptattn_bwd_noalloc(*[ctypes.c_void_p(x) for x in p], B, H, T, D, scale, None)


def test_noalloc_rejects_bad_arguments_before_any_hip_call(lib):
    """The no-allocation backward validates like gptattn_bwd (minus the
    workspace), and refuses B*H*T beyond its fixed scratch array, all
    before touching the HIP runtime."""
    text = open(HEADER).read()
    limit = int(re.search(r"GPTATTN_NOALLOC_MAX_ROWS\s+(\d+)", text).group(1))
    assert limit == G.NOALLOC_MAX_ROWS == 1 << 20
    assert bwd_noalloc(lib, B=1, H=16, T=limit // 16 + 1) == SCRATCH
    assert bwd_noalloc(lib, B=3, H=(limit + 2) // 3, T=1) == SCRATCH
    assert bwd_noalloc(lib, D=96) == UNSUPPORTED
    assert bwd_noalloc(lib, scale=float("nan")) == INVALID
    p = list(A[:9])
    p[6] = 0
    assert bwd_noalloc(lib, p) == INVALID
    p = list(A[:9])
    p[7] = p[6]
    assert bwd_noalloc(lib, p) == INVALID
    assert "SCRATCH" in G.status_string(SCRATCH)
