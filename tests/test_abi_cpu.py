"""CPU-side checks of the C-ABI library: it loads, exports every function
include/f8lin.h declares, and rejects bad arguments before launching anything
(these calls return from host-side validation and touch no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "libf8lin.so")
HEADER_DIR = os.path.join(ROOT, "include")

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE = 0, 1, 2, 3, 4


def _declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(f8lin_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libf8lin.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("f8lin_amax", "f8lin_cast_transpose", "f8lin_forward", "f8lin_backward",
                     "f8lin_delayed_update", "f8lin_gemm", "f8lin_gemm_batch", "f8lin_cast_f32", "f8lin_workspace_bytes",
                     "f8lin_dbias_workspace_bytes", "f8lin_backward_gemm_workspace_bytes",
                     "f8lin_status_str"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_workspace_and_status_strings(lib):
    lib.f8lin_workspace_bytes.restype = ctypes.c_size_t
    assert 4096 <= lib.f8lin_workspace_bytes() <= WSB
    lib.f8lin_status_str.restype = ctypes.c_char_p
    lib.f8lin_status_str.argtypes = [ctypes.c_int]
    for code in range(6):
        assert lib.f8lin_status_str(code).startswith(b"F8LIN_")
    assert b"unknown" in lib.f8lin_status_str(99)


class State(ctypes.Structure):
    _fields_ = [("amax", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("history", ctypes.c_void_p),
                ("hist_meta", ctypes.c_void_p)]


# Fake, never-dereferenced addresses: validation rejects before any launch.
A = 0x10000000
B = 0x20000000
C = 0x30000000
WS = 0x40000000
AMAX = 0x50000000
SCALE = 0x50000100
HIST = 0x50000200
META = 0x50000300
WSB = 1 << 20  # a workspace size above f8lin_workspace_bytes()


def test_amax_rejections(lib):
    f = lib.f8lin_amax
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(A, 64, 0, None, WS, WSB, None) == EINVAL          # no output
    assert f(None, 64, 0, AMAX, WS, WSB, None) == EINVAL       # no input with elements
    assert f(A, 64, 2, AMAX, WS, WSB, None) == EINVAL          # bad algorithm
    assert f(A, -1, 0, AMAX, WS, WSB, None) == ESHAPE
    assert f(A + 2, 64, 0, AMAX, WS, WSB, None) == EALIGN
    assert f(A, 64, 0, AMAX, None, WSB, None) == EWORKSPACE
    assert f(A, 64, 0, AMAX, WS, 16, None) == EWORKSPACE
    assert f(A, 64, 1, AMAX, WS + 8, WSB, None) == EWORKSPACE   # misaligned workspace
    assert f(A, 64, 0, A + 16, WS, WSB, None) == EINVAL       # output inside the input


def test_cast_rejections(lib):
    f = lib.f8lin_cast_transpose
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(State), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    st = State(AMAX, SCALE, None, None)
    dst = State(AMAX, SCALE, HIST, META)
    assert f(A, 32, 48, 0, 0, None, B, C, None) == EINVAL        # no state
    assert f(A, 32, 48, 2, 0, ctypes.byref(st), B, C, None) == EINVAL
    assert f(A, 32, 48, 0, 5, ctypes.byref(st), B, C, None) == EINVAL
    assert f(A, 32, 48, 0, 1, ctypes.byref(st), B, C, None) == EINVAL  # delayed without history
    assert f(A, 33, 48, 0, 0, ctypes.byref(st), B, C, None) == ESHAPE
    assert f(A, 32, 40, 0, 0, ctypes.byref(st), B, C, None) == ESHAPE
    assert f(A, -16, 48, 0, 0, ctypes.byref(st), B, C, None) == ESHAPE
    assert f(A, 32, 48, 0, 0, ctypes.byref(st), B + 1, C, None) == EALIGN
    assert f(A, 32, 48, 0, 0, ctypes.byref(st), B, C + 8, None) == EALIGN
    assert f(A, 32, 48, 0, 0, ctypes.byref(st), B, B + 512, None) == EINVAL  # q and qt overlap
    assert f(A, 32, 48, 0, 0, ctypes.byref(st), A + 1024, C, None) == EINVAL  # q inside x
    bad = State(AMAX, AMAX, None, None)  # scale overlaps amax
    assert f(A, 32, 48, 0, 0, ctypes.byref(bad), B, C, None) == EINVAL
    assert f(None, 32, 48, 0, 1, ctypes.byref(dst), B, C, None) == EINVAL


def test_gemm_rejections(lib):
    f = lib.f8lin_gemm
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(A, 0, B, 0, 32, 48, 64, None, SCALE, C, None) == EINVAL
    assert f(A, 0, B, 3, 32, 48, 64, AMAX, SCALE, C, None) == EINVAL
    assert f(A, 0, B, 0, 32, 48, 65, AMAX, SCALE, C, None) == ESHAPE
    assert f(A, 0, B, 0, 1 << 31, 48, 64, AMAX, SCALE, C, None) == ESHAPE
    assert f(A, 0, B + 4, 0, 32, 48, 64, AMAX, SCALE, C, None) == EALIGN
    assert f(A, 0, B, 0, 32, 48, 64, AMAX, SCALE, A, None) == EINVAL   # C aliases A
    assert f(None, 0, B, 0, 32, 48, 64, AMAX, SCALE, C, None) == EINVAL


def test_transposed_row_stride(lib):
    """Transposed copies whose rows hold a multiple of 32768 codes get 128
    bytes of padding per row; every other length is unpadded."""
    f = lib.f8lin_transposed_ld
    f.argtypes = [ctypes.c_int64]
    f.restype = ctypes.c_int64
    for n, want in ((0, 0), (16, 16), (4096, 4096), (16384, 16384), (32752, 32752), (32768, 32896),
                    (65536, 65664), (98304, 98432), (1 << 22, (1 << 22) + 128), (-16, 0)):
        assert f(n) == want, n


class GemmDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("a", "b", "inv_scale_a", "inv_scale_b", "c")] + \
               [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("lda", ctypes.c_int64),
                ("ldb", ctypes.c_int64)]


def test_gemm_batch_rejections(lib):
    f = lib.f8lin_gemm_batch
    f.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    C2 = C + (1 << 20)
    ok0 = GemmDesc(A, B, AMAX, SCALE, C, 32, 48, 64)
    ok1 = GemmDesc(B, A, AMAX, SCALE, C2, 48, 32, 64)
    arr = (GemmDesc * 5)(ok0, ok1, ok0, ok1, ok0)
    assert f(None, 1, 0, 0, None) == EINVAL
    assert f(arr, 0, 0, 0, None) == EINVAL                      # empty batch
    assert f(arr, 5, 0, 0, None) == EINVAL                      # more than F8LIN_MAX_BATCH
    assert f(arr, 3, 0, 0, None) == EINVAL                      # entries 0 and 2 write the same C
    assert f(arr, 2, 0, 4, None) == EINVAL                      # bad format
    bad = (GemmDesc * 2)(ok0, GemmDesc(B, A, AMAX, SCALE, C2, 48, 32, 65))
    assert f(bad, 2, 0, 0, None) == ESHAPE                      # second entry's K not a multiple of 16
    bad = (GemmDesc * 2)(ok0, GemmDesc(B, A, AMAX, SCALE, C2 + 4, 48, 32, 64))
    assert f(bad, 2, 0, 0, None) == EALIGN
    bad = (GemmDesc * 2)(ok0, GemmDesc(B, A, AMAX, SCALE, C + 64, 48, 32, 64))
    assert f(bad, 2, 0, 0, None) == EINVAL                      # the two outputs overlap
    bad = (GemmDesc * 2)(ok0, GemmDesc(B, C, AMAX, SCALE, C2, 48, 32, 64))
    assert f(bad, 2, 0, 0, None) == EINVAL                      # second input is the first output
    # row strides: 0 means K; otherwise at least K and a multiple of 16, and the overlap checks use them
    assert f((GemmDesc * 1)(GemmDesc(A, B, AMAX, SCALE, C, 32, 48, 64, 48, 0)), 1, 0, 0, None) == ESHAPE  # lda < K
    assert f((GemmDesc * 1)(GemmDesc(A, B, AMAX, SCALE, C, 32, 48, 64, 0, 72)), 1, 0, 0, None) == ESHAPE  # not x16
    assert f((GemmDesc * 1)(GemmDesc(A, B, AMAX, SCALE, A + 32 * 64 - 16, 32, 48, 64, 0, 0)), 1, 0, 0, None) == EINVAL
    # a strided A reaches further: C right after A's unstrided bytes now overlaps it
    assert f((GemmDesc * 1)(GemmDesc(A, B, AMAX, SCALE, A + 32 * 64 + 4096, 32, 48, 64, 256, 0)), 1, 0, 0,
             None) == EINVAL


class Fwd(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)] + \
               [(n, ctypes.c_void_p) for n in ("x", "w", "y", "x8", "x8t", "w8", "w8t")] + \
               [("sx", State), ("sw", State), ("mode_x", ctypes.c_int), ("mode_w", ctypes.c_int),
                ("algo", ctypes.c_int), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("bias", ctypes.c_void_p), ("w_cast_valid", ctypes.c_int), ("ev_gemm_begin", ctypes.c_void_p),
                ("ev_gemm_end", ctypes.c_void_p), ("y_amax", ctypes.c_void_p), ("x_amax_given", ctypes.c_int)]


class Bwd(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)] + \
               [(n, ctypes.c_void_p) for n in ("dy", "x8t", "w8t", "dx", "dw", "dy8", "dy8t")] + \
               [("sx", State), ("sw", State), ("sdy", State), ("mode_dy", ctypes.c_int), ("algo", ctypes.c_int),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("dbias", ctypes.c_void_p),
                ("dbias_ws", ctypes.c_void_p), ("dbias_ws_bytes", ctypes.c_size_t), ("gemm_ws", ctypes.c_void_p),
                ("gemm_ws_bytes", ctypes.c_size_t), ("ev_gemm_begin", ctypes.c_void_p), ("ev_gemm_end", ctypes.c_void_p),
                ("dx_amax", ctypes.c_void_p), ("dy_amax_given", ctypes.c_int)]


def test_backward_rejections(lib):
    f = lib.f8lin_backward
    f.argtypes = [ctypes.POINTER(Bwd), ctypes.c_void_p]
    f.restype = ctypes.c_int
    g = lib.f8lin_dbias_workspace_bytes
    g.argtypes = [ctypes.c_int64, ctypes.c_int64]
    g.restype = ctypes.c_size_t
    assert g(300, 48) == 3 * 48 * 4 and g(0, 48) == 48 * 4 and g(128, 16) == 64
    MB = 1 << 20
    DB = A + 9 * MB
    DBWS = A + 10 * MB

    def args(**kw):
        a = Bwd(288, 48, 64, A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB, A + 6 * MB,
                State(AMAX, SCALE, None, None), State(AMAX + 64, SCALE + 64, None, None),
                State(AMAX + 128, SCALE + 128, None, None), 0, 0, WS, WSB, None, None, 0, None, 0)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    need = g(288, 48)
    assert f(None, None) == EINVAL
    assert f(ctypes.byref(args(N=40)), None) == ESHAPE
    assert f(ctypes.byref(args(dbias=DB)), None) == EWORKSPACE                          # dbias without scratch
    assert f(ctypes.byref(args(dbias=DB, dbias_ws=DBWS, dbias_ws_bytes=need - 4)), None) == EWORKSPACE
    assert f(ctypes.byref(args(dbias=DB + 2, dbias_ws=DBWS, dbias_ws_bytes=need)), None) == EALIGN
    assert f(ctypes.byref(args(dbias=DB, dbias_ws=A, dbias_ws_bytes=need)), None) == EINVAL  # scratch is dY
    assert f(ctypes.byref(args(dbias=A + MB, dbias_ws=DBWS, dbias_ws_bytes=need)), None) == EINVAL  # dbias in x8t
    # amax of dX from the epilogue: a 4-byte aligned word outside every other buffer
    assert f(ctypes.byref(args(dx_amax=AMAX + 256 + 2)), None) == EALIGN
    assert f(ctypes.byref(args(dx_amax=A + 3 * MB + 64)), None) == EINVAL                  # inside dX
    assert f(ctypes.byref(args(dx_amax=SCALE + 128)), None) == EINVAL                       # dY's scale
    # dY's amax handed in: dynamic mode only
    assert f(ctypes.byref(args(dy_amax_given=1, mode_dy=1, sdy=State(AMAX + 128, SCALE + 128, HIST, META))),
             None) == EINVAL


def test_backward_gemm_workspace(lib):
    """Split-GEMM scratch: its size query, and a misaligned or overlapping
    gemm_ws is rejected (every call here fails validation: nothing runs)."""
    g = lib.f8lin_backward_gemm_workspace_bytes
    g.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    g.restype = ctypes.c_size_t
    # dW of a 256 x 256 weight over 4096 tokens: one output tile, 32 K blocks -> four K ranges of fp32 partials
    assert g(4096, 256, 256) == 4 * 256 * 256 * 4
    # dX (M, K) of a few rows with a long contraction over N splits too; square layers split nothing
    assert g(256, 4096, 256) == 4 * 256 * 256 * 4 + 0
    assert g(4096, 4096, 4096) == 0 and g(16, 4096, 4096) == 0
    assert g(4096, 4096, 4095) == 0 and g(-16, 16, 16) == 0  # invalid dimensions
    # the GPT-block output projection (1600 -> 1600 over 12288 tokens): dW splits five ways
    assert g(12288, 1600, 1600) == 5 * 1600 * 1600 * 4

    f = lib.f8lin_backward
    f.argtypes = [ctypes.POINTER(Bwd), ctypes.c_void_p]
    f.restype = ctypes.c_int
    SL = 16 << 20  # 16 MiB between fake buffers
    M, N, K = 4096, 256, 256
    need = g(M, N, K)

    def args(**kw):
        a = Bwd(M, N, K, A, A + SL, A + 2 * SL, A + 3 * SL, A + 4 * SL, A + 5 * SL, A + 6 * SL,
                State(AMAX, SCALE, None, None), State(AMAX + 64, SCALE + 64, None, None),
                State(AMAX + 128, SCALE + 128, None, None), 0, 0, WS, WSB, None, None, 0, None, 0)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    GW = A + 8 * SL
    assert f(ctypes.byref(args(gemm_ws=GW + 8, gemm_ws_bytes=need)), None) == EALIGN
    assert f(ctypes.byref(args(gemm_ws=A + 3 * SL, gemm_ws_bytes=need)), None) == EINVAL    # scratch is dX
    assert f(ctypes.byref(args(gemm_ws=A + SL - 4096, gemm_ws_bytes=need)), None) == EINVAL  # runs into x8t
    # with too little scratch only what fits would split, but overlap is checked on that part
    assert f(ctypes.byref(args(gemm_ws=A + 2 * SL, gemm_ws_bytes=64)), None) == EINVAL      # scratch is w8t


def test_forward_rejections(lib):
    f = lib.f8lin_forward
    f.argtypes = [ctypes.POINTER(Fwd), ctypes.c_void_p]
    f.restype = ctypes.c_int
    MB = 1 << 20

    def args(**kw):
        a = Fwd(32, 48, 64, A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB, A + 6 * MB,
                State(AMAX, SCALE, None, None), State(AMAX + 64, SCALE + 64, None, None), 0, 0, 0, WS, WSB)
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    assert f(None, None) == EINVAL
    assert f(ctypes.byref(args(K=63)), None) == ESHAPE
    assert f(ctypes.byref(args(mode_w=7)), None) == EINVAL
    assert f(ctypes.byref(args(y=A + 2 * MB + 2)), None) == EALIGN
    assert f(ctypes.byref(args(ws_bytes=100)), None) == EWORKSPACE
    assert f(ctypes.byref(args(w8=A + 3 * MB)), None) == EINVAL  # w8 aliases x8
    assert f(ctypes.byref(args(sw=State(AMAX, SCALE + 64, None, None))), None) == EINVAL  # shared amax slot
    assert f(ctypes.byref(args(mode_x=1)), None) == EINVAL  # delayed without history
    assert f(ctypes.byref(args(bias=A + 9 * MB + 2)), None) == EALIGN
    assert f(ctypes.byref(args(bias=A + 2 * MB)), None) == EINVAL  # bias inside Y
    # a reused weight cast: w is not read (null allowed), but w8 / w8t / scale must be there
    assert f(ctypes.byref(args(w_cast_valid=1, w=None, sw=State(AMAX + 64, None, None, None))), None) == EINVAL
    assert f(ctypes.byref(args(w_cast_valid=1, w=None, w8=None)), None) == EINVAL
    # amax of Y from the epilogue, and X's amax handed in
    assert f(ctypes.byref(args(y_amax=AMAX + 256 + 1)), None) == EALIGN
    assert f(ctypes.byref(args(y_amax=A + 2 * MB + 32)), None) == EINVAL                    # inside Y
    assert f(ctypes.byref(args(y_amax=AMAX)), None) == EINVAL                               # X's own amax word
    assert f(ctypes.byref(args(x_amax_given=1, mode_x=1, sx=State(AMAX, SCALE, HIST, META))), None) == EINVAL
    # X's amax is read, not written, when handed in: still no output may cover it
    assert f(ctypes.byref(args(x_amax_given=1, y_amax=AMAX)), None) == EINVAL
    # shared X: every entry must agree on X and its state
    g = lib.f8lin_forward_shared_x
    g.argtypes = [ctypes.POINTER(Fwd), ctypes.c_int, ctypes.c_void_p]
    g.restype = ctypes.c_int
    e1 = args(w=A + 7 * MB, y=A + 8 * MB, w8=A + 9 * MB, w8t=A + 10 * MB, sw=State(AMAX + 128, SCALE + 128, None, None))
    pair = (Fwd * 2)(args(), e1)
    assert g(pair, 0, None) == EINVAL
    assert g(pair, 5, None) == EINVAL
    bad = (Fwd * 2)(args(), args(w=A + 7 * MB, y=A + 8 * MB, w8=A + 9 * MB, w8t=A + 10 * MB, x=A + 11 * MB,
                                 sw=State(AMAX + 128, SCALE + 128, None, None)))
    assert g(bad, 2, None) == EINVAL                                  # different X
    clash = (Fwd * 2)(args(), args(w=A + 7 * MB, w8=A + 9 * MB, w8t=A + 10 * MB,
                                   sw=State(AMAX + 128, SCALE + 128, None, None)))
    assert g(clash, 2, None) == EINVAL                                # both write the same Y


def test_delayed_update_rejections(lib):
    f = lib.f8lin_delayed_update
    f.argtypes = [ctypes.POINTER(State), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    arr = (State * 2)(State(AMAX, SCALE, HIST, META), State(AMAX, SCALE, None, META))
    assert f(arr, 2, None, None) == EINVAL
    assert f(arr, -1, None, None) == EINVAL
    assert f(None, 1, None, None) == EINVAL
    arr2 = (State * 1)(State(AMAX, SCALE, HIST + 4, META))
    assert f(arr2, 1, None, None) == EALIGN
    ok = (State * 1)(State(AMAX, SCALE, HIST, META))
    assert f(ok, 1, C + 2, None) == EALIGN         # status words are int32
    assert f(ok, 1, HIST + 8, None) == EINVAL      # status inside the history
    assert f(ok, 1, META + 4, None) == EINVAL      # status inside {count, pos}
