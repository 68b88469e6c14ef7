"""Python face of the oracle (test infrastructure only; see oracle/__init__.py).

All tensors are numpy arrays: bf16 tensors as their uint16 bit patterns, fp8
tensors as uint8 codes, row-major.  Shapes follow the linear layer
Y = X W^T:  X (M, K), W (N, K), dY (M, N).

Where each step comes from:
  * tensorwise dynamic scaling -- one scale per tensor from that tensor's
    current amax (pytorch/torchtitan PR #778, "Integrate float8nocompile",
    Summary and the single-linear-layer table's ATOMIC_MAX / REDUCTION rows,
    which compute the same amax two ways);
  * delayed scaling of input, weight and grad_output from an amax history,
    synced after backward (pytorch/ao issue #1297, repro script's
    Float8LinearConfig and its training loop);
  * the forward + backward of one linear layer as the measured unit
    (PR #778, "Benchmarking single linear layer forward+backward
    performance").
The formats (OCP E4M3 for X and W, E5M2 for dY), eps, and the order
"fp32 multiply, then saturating round-to-nearest-even" are readings: the pages
name fp8 training and tensorwise scaling but never write the arithmetic.
"""
import ctypes
import math
import os

import numpy as np

E4M3 = 0
E5M2 = 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}
HIST_LEN = 16
EPS = np.float32(1e-12)

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def _load():
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"oracle library {path} is not built; run `python oracle/build.py`")
    lib = ctypes.CDLL(path)
    c_u16p = ctypes.POINTER(ctypes.c_uint16)
    c_u8p = ctypes.POINTER(ctypes.c_uint8)
    c_f32p = ctypes.POINTER(ctypes.c_float)
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8, ctypes.c_int]
    lib.oracle_fp8_decode.restype = ctypes.c_double
    lib.oracle_fp8_encode.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.oracle_fp8_encode.restype = ctypes.c_uint8
    lib.oracle_amax.argtypes = [c_u16p, ctypes.c_int64]
    lib.oracle_amax.restype = ctypes.c_float
    lib.oracle_scale.argtypes = [ctypes.c_float, ctypes.c_int, c_f32p, c_f32p]
    lib.oracle_scale.restype = None
    lib.oracle_cast.argtypes = [c_u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                c_u8p, c_u8p]
    lib.oracle_cast.restype = ctypes.c_int64
    lib.oracle_encode_f32.argtypes = [c_f32p, ctypes.c_int64, ctypes.c_int, c_u8p]
    lib.oracle_encode_f32.restype = None
    lib.oracle_encode_bits_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, c_u8p]
    lib.oracle_encode_bits_range.restype = None
    lib.oracle_history_amax.argtypes = [c_f32p]
    lib.oracle_history_amax.restype = ctypes.c_float
    lib.oracle_history_push.argtypes = [c_f32p, c_i32p, c_i32p, ctypes.c_float]
    lib.oracle_history_push.restype = None
    return lib


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ----------------------------------------------------------------- scalars

def bf16_bits_to_f32(bits: int) -> float:
    return float(_lib().oracle_bf16_to_f32(int(bits)))


def fp8_decode_scalar(code: int, fmt: int) -> float:
    """Exact value of one fp8 code (OCP OFP8 encoding)."""
    return float(_lib().oracle_fp8_decode(int(code), int(fmt)))


def fp8_encode_scalar(v: float, fmt: int) -> int:
    """Saturating round-to-nearest-even encode of one binary32 value."""
    return int(_lib().oracle_fp8_encode(ctypes.c_float(v), int(fmt)))


_TABLES = {}


def decode_table(fmt: int) -> np.ndarray:
    """fp64 value of each of the 256 codes of `fmt` (NaN codes decode to NaN)."""
    if fmt not in _TABLES:
        _TABLES[fmt] = np.array([fp8_decode_scalar(c, fmt) for c in range(256)], dtype=np.float64)
    return _TABLES[fmt]


def decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    return decode_table(fmt)[codes]


# ------------------------------------------------------------ element-wise

def amax(x_bits: np.ndarray) -> np.float32:
    """max |x| over a bf16 tensor (0 for an empty tensor, NaN if any NaN)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
    return np.float32(_lib().oracle_amax(_ptr(x, ctypes.c_uint16), x.size))


def scale(a, fmt: int):
    """(scale, inverse scale) = (fmax / max(amax, eps), 1 / scale), binary32."""
    s = ctypes.c_float()
    inv = ctypes.c_float()
    _lib().oracle_scale(ctypes.c_float(float(a)), int(fmt), ctypes.byref(s), ctypes.byref(inv))
    return np.float32(s.value), np.float32(inv.value)


def cast(x_bits: np.ndarray, fmt: int, s, transpose: bool = True):
    """fp8 codes of fl32(x * s) (saturating RNE), its transposed copy and the
    number of saturated elements.  x_bits is a 2-D uint16 (rows, cols)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    assert x.ndim == 2
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    qt = np.empty((cols, rows), dtype=np.uint8) if transpose else None
    nsat = _lib().oracle_cast(_ptr(x, ctypes.c_uint16), rows, cols, int(fmt), ctypes.c_float(float(s)),
                              _ptr(q, ctypes.c_uint8),
                              _ptr(qt, ctypes.c_uint8) if transpose else None)
    return q, qt, int(nsat)


def encode_f32(v: np.ndarray, fmt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_encode_f32(_ptr(v, ctypes.c_float), v.size, int(fmt), _ptr(q, ctypes.c_uint8))
    return q


def encode_bits_range(lo: int, count: int, fmt: int) -> np.ndarray:
    """Codes for the fp32 bit patterns lo, lo+1, ..., lo+count-1."""
    q = np.empty(count, dtype=np.uint8)
    _lib().oracle_encode_bits_range(ctypes.c_uint32(lo), ctypes.c_uint32(count), int(fmt),
                                    _ptr(q, ctypes.c_uint8))
    return q


# ------------------------------------------------------------------ GEMMs
# Y = X W^T, dX = dY W, dW = dY^T X on the dequantised fp8 tensors: each code
# decodes exactly to fp64, each product of two fp8 values is exact in fp64,
# the sums are fp64, and the result is divided by both tensor scales.

def gemm_ref(a8, fmt_a, b8, fmt_b, sa, sb):
    """C (M, N) = (A8 . B8^T) / (s_a s_b) for fp8 codes A8 (M, K) in format
    fmt_a and B8 (N, K) in fmt_b, both laid out along K (the one product all
    three GEMMs of the layer are instances of, given the transposed copies)."""
    a = decode(a8, fmt_a)
    b = decode(b8, fmt_b)
    return (a @ b.T) / np.float64(sa) / np.float64(sb)


def forward_ref(x8, w8, sx, sw, bias_bits=None):
    """Y (M, N) = (X8 . W8^T) / (s_x s_w) [+ b], X8 (M, K) e4m3, W8 (N, K) e4m3,
    b (N,) bf16 bits added to every row."""
    a = decode(x8, E4M3)
    b = decode(w8, E4M3)
    y = (a @ b.T) / np.float64(sx) / np.float64(sw)
    if bias_bits is not None:
        y = y + bf16_to_f64(bias_bits)[None, :]
    return y


def dgrad_ref(dy8, w8, sdy, sw):
    """dX (M, K) = (dY8 . W8) / (s_dy s_w), dY8 (M, N) e5m2, W8 (N, K) e4m3."""
    a = decode(dy8, E5M2)
    b = decode(w8, E4M3)
    return (a @ b) / np.float64(sdy) / np.float64(sw)


def wgrad_ref(dy8, x8, sdy, sx):
    """dW (N, K) = (dY8^T . X8) / (s_dy s_x), dY8 (M, N) e5m2, X8 (M, K) e4m3."""
    a = decode(dy8, E5M2)
    b = decode(x8, E4M3)
    return (a.T @ b) / np.float64(sdy) / np.float64(sx)


def _dot_rows(a_rows: np.ndarray, b_rows: np.ndarray) -> np.ndarray:
    # Row-by-row fp64 dot products: sum_k a[r, k] * b[r, k].
    return np.einsum("rk,rk->r", a_rows, b_rows)


def forward_ref_at(x8, w8, sx, sw, rows, cols):
    """Y[rows[i], cols[i]] for sampled entries (same definition as forward_ref)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = decode(x8[rows, :], E4M3)
    b = decode(w8[cols, :], E4M3)
    return _dot_rows(a, b) / np.float64(sx) / np.float64(sw)


def dgrad_ref_at(dy8, w8, sdy, sw, rows, cols):
    """dX[rows[i], cols[i]] = sum_n dY8[r, n] W8[n, c] / (s_dy s_w)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = decode(dy8[rows, :], E5M2)
    b = decode(np.ascontiguousarray(w8[:, cols].T), E4M3)
    return _dot_rows(a, b) / np.float64(sdy) / np.float64(sw)


def wgrad_ref_at(dy8, x8, sdy, sx, rows, cols):
    """dW[rows[i], cols[i]] = sum_m dY8[m, r] X8[m, c] / (s_dy s_x)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = decode(np.ascontiguousarray(dy8[:, rows].T), E5M2)
    b = decode(np.ascontiguousarray(x8[:, cols].T), E4M3)
    return _dot_rows(a, b) / np.float64(sdy) / np.float64(sx)


# -------------------------------------------------------------------- bias
# The linear layers of the GPT-1.5B repro carry a bias (pytorch/ao issue
# #1297, repro script: the nn.Linear layers of CausalSelfAttention and
# GPTBlock keep nn.Linear's default bias).  Such a layer computes
# Y = X W^T + b, and its backward produces the bias gradient: the sum of dY
# over the token rows.  Both are written out from that definition; the bias
# and its gradient stay in bf16 (reading: the pages cast only the three GEMM
# operands to fp8).

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dbias_ref(dy_bits: np.ndarray) -> np.ndarray:
    """db[n] = sum over rows m of dY[m, n], in fp64 (dY (M, N) bf16 bits)."""
    d = bf16_to_f64(dy_bits)
    out = np.zeros(d.shape[1], dtype=np.float64)
    for m in range(d.shape[0]):  # rows in order: a plain running sum per column
        out += d[m]
    return out


# --------------------------------------------------------- delayed scaling

class DelayedHistory:
    """Amax history of one tensor role for delayed scaling.

    The scale of a step comes from the largest amax of the *previous* steps
    (the history is only updated after backward, by the sync call).  The
    first step of a role has no history: it takes its scale from the current
    tensor's amax (the amax-initialisation the repro's config toggles)."""

    def __init__(self):
        self.hist = np.zeros(HIST_LEN, dtype=np.float32)
        self.count = 0
        self.pos = 0

    def amax_for_scale(self, x_bits):
        if self.count == 0:
            return amax(x_bits)
        return np.float32(_lib().oracle_history_amax(_ptr(self.hist, ctypes.c_float)))

    def push(self, amax_now):
        count = ctypes.c_int32(self.count)
        pos = ctypes.c_int32(self.pos)
        _lib().oracle_history_push(_ptr(self.hist, ctypes.c_float), ctypes.byref(count), ctypes.byref(pos),
                                   ctypes.c_float(float(amax_now)))
        self.count, self.pos = count.value, pos.value

    def copy(self):
        h = DelayedHistory()
        h.hist = self.hist.copy()
        h.count = self.count
        h.pos = self.pos
        return h


def _quantize(t_bits, fmt, amax_for_scale=None):
    a_now = amax(t_bits)
    a = a_now if amax_for_scale is None else np.float32(amax_for_scale)
    s, inv = scale(a, fmt)
    q, qt, nsat = cast(t_bits, fmt, s)
    return {"amax": a_now, "scale": s, "inv_scale": inv, "q": q, "qt": qt, "saturated": nsat}


def linear_step(x_bits, w_bits, dy_bits, *, amax_x=None, amax_w=None, amax_dy=None, gemms=True,
                bias_bits=None):
    """One forward + backward of a tensorwise-scaled Float8Linear.

    amax_* override the amax a tensor's scale is computed from (delayed
    scaling passes the history's amax); None means dynamic scaling.  Returns
    the per-tensor results and, if `gemms`, the fp64 Y, dX and dW.  With a
    bias (bf16 bits, (N,)), Y includes it and "dbias" holds its gradient."""
    qx = _quantize(x_bits, E4M3, amax_x)
    qw = _quantize(w_bits, E4M3, amax_w)
    qdy = _quantize(dy_bits, E5M2, amax_dy)
    out = {"x": qx, "w": qw, "dy": qdy}
    if gemms:
        out["y"] = forward_ref(qx["q"], qw["q"], qx["scale"], qw["scale"], bias_bits)
        out["dx"] = dgrad_ref(qdy["q"], qw["q"], qdy["scale"], qw["scale"])
        out["dw"] = wgrad_ref(qdy["q"], qx["q"], qdy["scale"], qx["scale"])
    if bias_bits is not None:
        out["dbias"] = dbias_ref(dy_bits)
    return out


__all__ = [n for n in dir() if not n.startswith("_")]
