"""Thin Python binding of libf8lin.so (include/f8lin.h), same names as the C ABI.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and streams; this module
checks dtypes / devices / contiguity, passes raw pointers and the current HIP
stream, and raises F8linError on a non-zero status.  Importing it fails
loudly if the library is not built -- there is no fallback.
"""
import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libf8lin.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                      "from the repository root")

_lib = ctypes.CDLL(LIB_PATH)

E4M3 = 0
E5M2 = 1
AMAX_ATOMIC = 0
AMAX_TWOPASS = 1
DYNAMIC = 0
DELAYED = 1
HISTORY_LEN = 16

_FMT = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
_ALGO = {"atomic": AMAX_ATOMIC, "twopass": AMAX_TWOPASS, AMAX_ATOMIC: AMAX_ATOMIC, AMAX_TWOPASS: AMAX_TWOPASS}
_MODE = {"dynamic": DYNAMIC, "delayed": DELAYED, DYNAMIC: DYNAMIC, DELAYED: DELAYED}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


class State(ctypes.Structure):
    _fields_ = [("amax", _vp), ("scale", _vp), ("history", _vp), ("hist_meta", _vp)]


class GemmDesc(ctypes.Structure):
    _fields_ = [("a", _vp), ("b", _vp), ("inv_scale_a", _vp), ("inv_scale_b", _vp), ("c", _vp),
                ("M", _i64), ("N", _i64), ("K", _i64), ("lda", _i64), ("ldb", _i64)]


MAX_BATCH = 4


class FwdArgs(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("x", _vp), ("w", _vp), ("y", _vp),
                ("x8", _vp), ("x8t", _vp), ("w8", _vp), ("w8t", _vp), ("sx", State), ("sw", State),
                ("mode_x", _int), ("mode_w", _int), ("algo", _int), ("ws", _vp), ("ws_bytes", ctypes.c_size_t),
                ("bias", _vp), ("w_cast_valid", _int), ("ev_gemm_begin", _vp), ("ev_gemm_end", _vp),
                ("y_amax", _vp), ("x_amax_given", _int)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64), ("dy", _vp), ("x8t", _vp), ("w8t", _vp),
                ("dx", _vp), ("dw", _vp), ("dy8", _vp), ("dy8t", _vp), ("sx", State), ("sw", State),
                ("sdy", State), ("mode_dy", _int), ("algo", _int), ("ws", _vp), ("ws_bytes", ctypes.c_size_t),
                ("dbias", _vp), ("dbias_ws", _vp), ("dbias_ws_bytes", ctypes.c_size_t), ("gemm_ws", _vp),
                ("gemm_ws_bytes", ctypes.c_size_t), ("ev_gemm_begin", _vp), ("ev_gemm_end", _vp),
                ("dx_amax", _vp), ("dy_amax_given", _int)]


_lib.f8lin_transposed_ld.argtypes = [_i64]
_lib.f8lin_transposed_ld.restype = _i64
_lib.f8lin_workspace_bytes.argtypes = []
_lib.f8lin_workspace_bytes.restype = ctypes.c_size_t
_lib.f8lin_dbias_workspace_bytes.argtypes = [_i64, _i64]
_lib.f8lin_dbias_workspace_bytes.restype = ctypes.c_size_t
_lib.f8lin_backward_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.f8lin_backward_gemm_workspace_bytes.restype = ctypes.c_size_t
_lib.f8lin_status_str.argtypes = [_int]
_lib.f8lin_status_str.restype = ctypes.c_char_p
_lib.f8lin_amax.argtypes = [_vp, _i64, _int, _vp, _vp, ctypes.c_size_t, _vp]
_lib.f8lin_cast_transpose.argtypes = [_vp, _i64, _i64, _int, _int, ctypes.POINTER(State), _vp, _vp, _vp]
_lib.f8lin_cast_f32.argtypes = [_vp, _i64, _int, _vp, _vp]
_lib.f8lin_gemm.argtypes = [_vp, _int, _vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
_lib.f8lin_gemm_batch.argtypes = [ctypes.POINTER(GemmDesc), _int, _int, _int, _vp]
_lib.f8lin_forward.argtypes = [ctypes.POINTER(FwdArgs), _vp]
_lib.f8lin_forward_shared_x.argtypes = [ctypes.POINTER(FwdArgs), _int, _vp]
_lib.f8lin_backward.argtypes = [ctypes.POINTER(BwdArgs), _vp]
_lib.f8lin_backward_noalloc.argtypes = [ctypes.POINTER(BwdArgs), _vp]
_lib.f8lin_delayed_update.argtypes = [ctypes.POINTER(State), _int, _vp, _vp]
for _name in ("f8lin_amax", "f8lin_cast_transpose", "f8lin_cast_f32", "f8lin_gemm", "f8lin_forward",
              "f8lin_backward", "f8lin_backward_noalloc", "f8lin_delayed_update"):
    getattr(_lib, _name).restype = _int


class F8linError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(_lib.f8lin_status_str(status).decode())


def _check(status: int):
    if status != 0:
        raise F8linError(status)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("f8lin: tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("f8lin: tensors must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"f8lin: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def transposed_ld(rows: int) -> int:
    """Row stride (bytes) of the transposed fp8 copy of a tensor with `rows` rows."""
    return int(_lib.f8lin_transposed_ld(rows))


def new_transposed(cols: int, rows: int, device="cuda") -> torch.Tensor:
    """A (cols, rows) uint8 tensor laid out as the library's transposed copies
    are: a view into a (cols, transposed_ld(rows)) buffer (uninitialised)."""
    ld = transposed_ld(rows)
    buf = torch.empty((cols, ld), dtype=torch.uint8, device=device)
    return buf[:, :rows] if ld != rows else buf


def _ptr_t(t: Optional[torch.Tensor]) -> Optional[int]:
    """Pointer of a transposed fp8 copy: a (cols, rows) uint8 tensor whose rows
    are transposed_ld(rows) bytes apart (see new_transposed)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("f8lin: tensors must be on the GPU")
    if t.dtype != torch.uint8 or t.dim() != 2:
        raise TypeError("f8lin: a transposed fp8 copy is a 2-D uint8 tensor")
    if t.numel() > 0 and (t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) != transposed_ld(t.shape[1]))):
        raise ValueError(f"f8lin: a transposed copy with rows of {t.shape[1]} codes needs a row stride of "
                         f"{transposed_ld(t.shape[1])} bytes (allocate it with new_transposed)")
    return t.data_ptr()


def _ptr_ld(t: torch.Tensor):
    """(pointer, row stride) of a 2-D uint8 GEMM operand whose rows are contiguous."""
    if not t.is_cuda:
        raise ValueError("f8lin: tensors must be on the GPU")
    if t.dtype != torch.uint8 or t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise TypeError("f8lin: a GEMM operand is a 2-D uint8 tensor with contiguous rows")
    return t.data_ptr(), (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def workspace_bytes() -> int:
    return int(_lib.f8lin_workspace_bytes())


def dbias_workspace_bytes(M: int, N: int) -> int:
    return int(_lib.f8lin_dbias_workspace_bytes(M, N))


def backward_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.f8lin_backward_gemm_workspace_bytes(M, N, K))


def new_backward_gemm_workspace(M: int, N: int, K: int, device="cuda") -> Optional[torch.Tensor]:
    """Scratch for split backward GEMMs (uninitialised), or None when no GEMM of this shape splits."""
    n = backward_gemm_workspace_bytes(M, N, K)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def new_dbias_workspace(M: int, N: int, device="cuda") -> torch.Tensor:
    """Scratch (float32, no initialisation needed) for the bias gradient of an (M, N) dY."""
    return torch.empty(max(1, dbias_workspace_bytes(M, N) // 4), dtype=torch.float32, device=device)


def status_str(status: int) -> str:
    return _lib.f8lin_status_str(status).decode()


def new_workspace(device="cuda") -> torch.Tensor:
    """A zero-filled workspace (uint8) of workspace_bytes()."""
    return torch.zeros(workspace_bytes(), dtype=torch.uint8, device=device)


class ScalingState:
    """Device-resident scaling state of one tensor role (f8lin_state):
    amax [1] f32, scale [2] f32 = {scale, 1/scale}, history [16] f32,
    hist_meta [2] i32 = {count, pos}; all zero-initialised."""

    def __init__(self, device="cuda", tensors=None):
        """tensors: optional (amax, scale, history, hist_meta) tensors to wrap
        instead of allocating new ones (e.g. a module's buffers)."""
        if tensors is not None:
            self.amax, self.scale, self.history, self.hist_meta = tensors
            return
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        self.scale = torch.zeros(2, dtype=torch.float32, device=device)
        self.history = torch.zeros(HISTORY_LEN, dtype=torch.float32, device=device)
        self.hist_meta = torch.zeros(2, dtype=torch.int32, device=device)

    def c_struct(self) -> State:
        return State(self.amax.data_ptr(), self.scale.data_ptr(), self.history.data_ptr(), self.hist_meta.data_ptr())

    @property
    def inv_scale(self) -> torch.Tensor:
        return self.scale[1:2]

    def state_dict(self):
        """Host copies of the state (for checkpointing)."""
        return {k: getattr(self, k).detach().cpu().clone() for k in ("amax", "scale", "history", "hist_meta")}

    def load_state_dict(self, sd):
        for k in ("amax", "scale", "history", "hist_meta"):
            getattr(self, k).copy_(sd[k])


class ScaleView:
    """A state that only carries {scale, 1/scale} (what backward reads of the
    forward's X and W states), e.g. a snapshot taken at forward time."""

    def __init__(self, scale: torch.Tensor):
        if scale.numel() != 2 or scale.dtype != torch.float32 or not scale.is_contiguous():
            raise ValueError("ScaleView needs a contiguous float32 tensor of 2 elements")
        self.scale = scale

    def c_struct(self) -> State:
        return State(None, self.scale.data_ptr(), None, None)


# ----------------------------------------------------------------- entry points

def amax(x: torch.Tensor, out: torch.Tensor, ws: torch.Tensor, algo="atomic", stream=None):
    _check(_lib.f8lin_amax(_ptr(x, torch.bfloat16), x.numel(), _ALGO[algo], _ptr(out, torch.float32),
                           _ptr(ws), _nbytes(ws), _stream(stream)))


def cast_transpose(x: torch.Tensor, fmt, mode, state: ScalingState, q: torch.Tensor,
                   qt: Optional[torch.Tensor] = None, stream=None):
    if x.dim() != 2:
        raise ValueError("cast_transpose takes a 2-D tensor")
    st = state.c_struct()
    _check(_lib.f8lin_cast_transpose(_ptr(x, torch.bfloat16), x.shape[0], x.shape[1], _FMT[fmt], _MODE[mode],
                                     ctypes.byref(st), _ptr(q, torch.uint8), _ptr_t(qt), _stream(stream)))


def cast_f32(v: torch.Tensor, fmt, q: torch.Tensor, stream=None):
    _check(_lib.f8lin_cast_f32(_ptr(v, torch.float32), v.numel(), _FMT[fmt], _ptr(q, torch.uint8),
                               _stream(stream)))


def gemm(a: torch.Tensor, fmt_a, b: torch.Tensor, fmt_b, inv_a: torch.Tensor, inv_b: torch.Tensor,
         c: torch.Tensor, stream=None):
    """c (M, N) bf16 = a (M, K) . b (N, K)^T * inv_a[0] * inv_b[0]."""
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or tuple(c.shape) != (M, N):
        raise ValueError("gemm: shape mismatch")
    _check(_lib.f8lin_gemm(_ptr(a, torch.uint8), _FMT[fmt_a], _ptr(b, torch.uint8), _FMT[fmt_b], M, N, K,
                           _ptr(inv_a, torch.float32), _ptr(inv_b, torch.float32), _ptr(c, torch.bfloat16),
                           _stream(stream)))


def gemm_batch(items, fmt_a, fmt_b, stream=None):
    """Up to MAX_BATCH GEMMs in one launch; items: (a, b, inv_a, inv_b, c) tuples
    as for gemm(), all with the operand formats fmt_a / fmt_b."""
    arr = (GemmDesc * max(1, len(items)))()
    for i, (a, b, inv_a, inv_b, c) in enumerate(items):
        M, K = a.shape
        N = b.shape[0]
        if b.shape[1] != K or tuple(c.shape) != (M, N):
            raise ValueError("gemm_batch: shape mismatch")
        pa, lda = _ptr_ld(a)
        pb, ldb = _ptr_ld(b)
        arr[i] = GemmDesc(pa, pb, _ptr(inv_a, torch.float32), _ptr(inv_b, torch.float32), _ptr(c, torch.bfloat16),
                          M, N, K, lda, ldb)
    _check(_lib.f8lin_gemm_batch(arr, len(items), _FMT[fmt_a], _FMT[fmt_b], _stream(stream)))


def _event(ev) -> Optional[int]:
    """Raw hipEvent_t of a torch.cuda.Event (created by recording it once), or None."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ev.cuda_event


def _amax_word(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() < 1:
        raise TypeError("f8lin: an amax output is a float32 tensor")
    return _ptr(t)


def _fwd_args(x, w, y, x8, x8t, w8, w8t, sx, sw, ws, mode_x, mode_w, algo, bias, w_cast_valid, gemm_events=None,
              y_amax=None, x_amax_given=False):
    M, K = x.shape
    N = w8.shape[0]
    if (w is not None and tuple(w.shape) != (N, K)) or tuple(w8.shape) != (N, K) or tuple(y.shape) != (M, N):
        raise ValueError("forward: shape mismatch")
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError("forward: bias must have shape (N,)")
    ev0, ev1 = (None, None) if gemm_events is None else gemm_events
    return FwdArgs(M, N, K, _ptr(x, torch.bfloat16), _ptr(w, torch.bfloat16), _ptr(y, torch.bfloat16),
                   _ptr(x8, torch.uint8), _ptr_t(x8t), _ptr(w8, torch.uint8), _ptr_t(w8t),
                   sx.c_struct(), sw.c_struct(), _MODE[mode_x], _MODE[mode_w], _ALGO[algo], _ptr(ws),
                   _nbytes(ws), None if bias is None else _ptr(bias, torch.bfloat16),
                   1 if w_cast_valid else 0, _event(ev0), _event(ev1), _amax_word(y_amax),
                   1 if x_amax_given else 0)


def forward(x, w, y, x8, x8t, w8, w8t, sx: ScalingState, sw: ScalingState, ws, mode_x="dynamic",
            mode_w="dynamic", algo="atomic", stream=None, bias=None, w_cast_valid=False, gemm_events=None,
            y_amax=None, x_amax_given=False):
    """w_cast_valid: w8, w8t and sw's scale already hold W's cast (unchanged
    weight); W's amax and cast are skipped and w may be None.
    gemm_events: optional (begin, end) torch.cuda.Event pair recorded around
    the call's GEMM launch.  y_amax: optional float32 tensor that receives
    amax(Y) from the GEMM epilogue.  x_amax_given: sx.amax already holds
    amax(X) (dynamic mode), so X's amax pass is skipped."""
    a = _fwd_args(x, w, y, x8, x8t, w8, w8t, sx, sw, ws, mode_x, mode_w, algo, bias, w_cast_valid, gemm_events,
                  y_amax, x_amax_given)
    _check(_lib.f8lin_forward(ctypes.byref(a), _stream(stream)))


def forward_shared_x(x, x8, x8t, sx: ScalingState, ws, linears, mode_x="dynamic", algo="atomic", stream=None,
                     gemm_events=None, x_amax_given=False):
    """Linears reading the same X: linears is a list of dicts with keys w, y,
    w8, w8t, sw and optionally mode_w, bias, w_cast_valid, y_amax.  X is cast
    once; the GEMMs share one launch."""
    arr = (FwdArgs * max(1, len(linears)))()
    for i, l in enumerate(linears):
        arr[i] = _fwd_args(x, l.get("w"), l["y"], x8, x8t, l["w8"], l["w8t"], sx, l["sw"], ws, mode_x,
                           l.get("mode_w", "dynamic"), algo, l.get("bias"), l.get("w_cast_valid", False),
                           gemm_events, l.get("y_amax"), x_amax_given)
    _check(_lib.f8lin_forward_shared_x(arr, len(linears), _stream(stream)))


def backward(dy, x8t, w8t, dx, dw, dy8, dy8t, sx: ScalingState, sw: ScalingState, sdy: ScalingState, ws,
             mode_dy="dynamic", algo="atomic", stream=None, dbias=None, dbias_ws=None, gemm_ws=None,
             gemm_events=None, dx_amax=None, dy_amax_given=False):
    """gemm_ws: optional scratch (backward_gemm_workspace_bytes(M, N, K) bytes) with which GEMMs that have
    few output tiles and a long contraction run split along K.  gemm_events, dx_amax, dy_amax_given: as
    forward's gemm_events, y_amax, x_amax_given, for the dgrad + wgrad launch, dX and dY."""
    M, N = dy.shape
    K = x8t.shape[0]
    if tuple(dx.shape) != (M, K) or tuple(dw.shape) != (N, K) or tuple(w8t.shape) != (K, N):
        raise ValueError("backward: shape mismatch")
    if dbias is not None and tuple(dbias.shape) != (N,):
        raise ValueError("backward: dbias must have shape (N,)")
    a = BwdArgs(M, N, K, _ptr(dy, torch.bfloat16), _ptr_t(x8t), _ptr_t(w8t),
                _ptr(dx, torch.bfloat16), _ptr(dw, torch.bfloat16), _ptr(dy8, torch.uint8), _ptr_t(dy8t),
                sx.c_struct(), sw.c_struct(), sdy.c_struct(), _MODE[mode_dy], _ALGO[algo], _ptr(ws),
                _nbytes(ws), None if dbias is None else _ptr(dbias, torch.bfloat16),
                None if dbias_ws is None else _ptr(dbias_ws, torch.float32),
                0 if dbias_ws is None else dbias_ws.numel() * 4, _ptr(gemm_ws), _nbytes(gemm_ws),
                *((None, None) if gemm_events is None else (_event(gemm_events[0]), _event(gemm_events[1]))),
                _amax_word(dx_amax), 1 if dy_amax_given else 0)
    _check(_lib.f8lin_backward(ctypes.byref(a), _stream(stream)))


def backward_noalloc(dy, x8t, w8t, dx, dw, dy8, dy8t, sx: ScalingState, sw: ScalingState, sdy: ScalingState,
                     mode_dy="dynamic", algo="atomic", stream=None, dbias=None, gemm_events=None, dx_amax=None,
                     dy_amax_given=False):
    """backward() for callers that cannot allocate: no workspace, bias-gradient
    scratch or split scratch is passed; the library's static per-device scratch
    (8 KB + 16 MiB) takes their place.  Calls that overlap in time on one GPU race."""
    M, N = dy.shape
    K = x8t.shape[0]
    if tuple(dx.shape) != (M, K) or tuple(dw.shape) != (N, K) or tuple(w8t.shape) != (K, N):
        raise ValueError("backward_noalloc: shape mismatch")
    if dbias is not None and tuple(dbias.shape) != (N,):
        raise ValueError("backward_noalloc: dbias must have shape (N,)")
    a = BwdArgs(M, N, K, _ptr(dy, torch.bfloat16), _ptr_t(x8t), _ptr_t(w8t),
                _ptr(dx, torch.bfloat16), _ptr(dw, torch.bfloat16), _ptr(dy8, torch.uint8), _ptr_t(dy8t),
                sx.c_struct(), sw.c_struct(), sdy.c_struct(), _MODE[mode_dy], _ALGO[algo], None, 0,
                None if dbias is None else _ptr(dbias, torch.bfloat16), None, 0, None, 0,
                *((None, None) if gemm_events is None else (_event(gemm_events[0]), _event(gemm_events[1]))),
                _amax_word(dx_amax), 1 if dy_amax_given else 0)
    _check(_lib.f8lin_backward_noalloc(ctypes.byref(a), _stream(stream)))


NOALLOC_REGION_BYTES = 16 << 20  # the static scratch's region for bias-gradient sums and split partials


def delayed_update(states: Sequence[ScalingState], stream=None, status: Optional[torch.Tensor] = None):
    """status: optional int32 device tensor of len(states); entry i becomes 0
    when state i was updated and 1 (F8LIN_EINVAL) when its {count, pos} was
    not a reachable one, in which case that state is left untouched."""
    arr = (State * max(1, len(states)))(*[s.c_struct() for s in states])
    if status is not None and (status.dtype != torch.int32 or status.numel() < len(states)):
        raise ValueError("delayed_update: status must be an int32 tensor of at least len(states) entries")
    _check(_lib.f8lin_delayed_update(arr, len(states), _ptr(status), _stream(stream)))


# ------------------------------------------------------------ layer buffers

class LinearBuffers:
    """Every device buffer one Float8Linear forward + backward needs, for
    X (M, K), W (N, K), dY (M, N); allocated once with torch (plumbing)."""

    def __init__(self, M: int, N: int, K: int, device="cuda", with_bias: bool = False):
        u8 = dict(dtype=torch.uint8, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.M, self.N, self.K = M, N, K
        self.y = torch.empty((M, N), **bf)
        self.dx = torch.empty((M, K), **bf)
        self.dw = torch.empty((N, K), **bf)
        self.x8 = torch.empty((M, K), **u8)
        self.x8t = new_transposed(K, M, device)
        self.w8 = torch.empty((N, K), **u8)
        self.w8t = new_transposed(K, N, device)
        self.dy8 = torch.empty((M, N), **u8)
        self.dy8t = new_transposed(N, M, device)
        self.sx = ScalingState(device)
        self.sw = ScalingState(device)
        self.sdy = ScalingState(device)
        self.ws = new_workspace(device)
        self.dbias = torch.empty((N,), **bf) if with_bias else None
        self.dbias_ws = new_dbias_workspace(M, N, device) if with_bias else None
        self.gemm_ws = new_backward_gemm_workspace(M, N, K, device)

    def forward(self, x, w, mode="dynamic", algo="atomic", stream=None, bias=None, gemm_events=None):
        forward(x, w, self.y, self.x8, self.x8t, self.w8, self.w8t, self.sx, self.sw, self.ws, mode, mode, algo,
                stream, bias, gemm_events=gemm_events)
        return self.y

    def backward(self, dy, mode="dynamic", algo="atomic", stream=None, gemm_events=None):
        backward(dy, self.x8t, self.w8t, self.dx, self.dw, self.dy8, self.dy8t, self.sx, self.sw, self.sdy,
                 self.ws, mode, algo, stream, self.dbias, self.dbias_ws, self.gemm_ws, gemm_events=gemm_events)
        return self.dx, self.dw

    def states(self):
        return [self.sx, self.sw, self.sdy]
