"""PyTorch module surface over the C ABI: a Float8Linear layer, the swap of
nn.Linear for it, and the delayed-scaling sync after backward.

This mirrors the user interface the pages show (pytorch/ao issue #1297,
repro script: convert_to_float8_training(model, config=Float8LinearConfig(
cast_config_input / weight / grad_output = CastConfig(ScalingType...))),
and sync_float8_amax_and_scale_history(model) after loss.backward();
pytorch/ao issue #1199: convert_to_float8_training swapping nn.Linear).
Every step of the forward and backward runs in libf8lin's HIP kernels;
this file only allocates tensors and marshals arguments.

Shapes: in_features and out_features must be multiples of 16.  The token
dimension may be anything: it is zero-padded to a multiple of 16, which is
exact (zero rows raise no amax, add nothing to dW or to the bias gradient,
and their Y / dX rows are dropped).  A bias (the repro's nn.Linear layers
keep theirs) is added in the GEMM epilogue and its gradient is summed in the
backward's cast pass.

Scaling state.  Each layer keeps, per tensor role (input x, weight w,
grad_output dy), the device state the library reads and writes -- amax,
{scale, 1/scale}, the 16-entry amax history and {count, pos} -- as
registered buffers, so model.state_dict() / load_state_dict() save and
restore it and model.to() moves it; which delayed roles have taken their
first step is saved as the module's extra state.

Delayed scaling, per role:
  * the scale comes from the largest amax of the previous steps (the
    history), and the cast folds this step's amax into the state;
  * a role's first step has no history: it takes its scale from the current
    tensor (amax initialisation).  It runs through the same delayed cast with
    a one-entry history seeded with the current tensor's amax (computed by
    the library's amax pass), so the scale is the dynamic one, bit for bit,
    and the state's amax still collects the maximum over every micro-batch
    of the step;
  * the sync after backward pushes the amax of every delayed role that has
    produced one since the last sync (a forward without backward produces
    none for dy), and only those roles count as initialised.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch
import torch.nn as nn

from . import f8lin

_ROLES = ("x", "w", "dy")
_STATE_FIELDS = (("amax", (1,), torch.float32), ("scale", (2,), torch.float32),
                 ("history", (f8lin.HISTORY_LEN,), torch.float32), ("hist_meta", (2,), torch.int32))


@dataclass
class CastConfig:
    scaling_type: str = "dynamic"  # "dynamic" or "delayed"

    def __post_init__(self):
        if self.scaling_type not in ("dynamic", "delayed"):
            raise ValueError(f"scaling_type must be 'dynamic' or 'delayed', got {self.scaling_type!r}")


@dataclass
class Float8LinearConfig:
    cast_config_input: CastConfig = field(default_factory=CastConfig)
    cast_config_weight: CastConfig = field(default_factory=CastConfig)
    cast_config_grad_output: CastConfig = field(default_factory=CastConfig)
    amax_algo: str = "twopass"  # "atomic" or "twopass"
    # Opt-in: reuse the weight's fp8 copies while the weight tensor and its
    # version counter are unchanged (e.g. the micro-batches of one optimizer
    # step).  Updates through .data (p.data.copy_, EMA, checkpoint loading)
    # do not move the version counter: after such an update call
    # invalidate_weight_cast(model).  The cache is also dropped at every
    # sync_float8_amax_and_scale_history.
    reuse_weight_cast: bool = False


def _pad_rows(t: torch.Tensor) -> torch.Tensor:
    m = t.shape[0]
    pad = (-m) % 16
    if pad == 0:
        return t.contiguous()
    return torch.cat([t, t.new_zeros((pad, t.shape[1]))], dim=0)


class _Float8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2d, weight, bias, layer):
        M0 = x2d.shape[0]
        x = _pad_rows(x2d.to(torch.bfloat16))
        b = None if bias is None else bias.to(torch.bfloat16).contiguous()
        M, K = x.shape
        N = weight.shape[0]
        dev = x.device
        u8 = dict(dtype=torch.uint8, device=dev)
        x8 = torch.empty((M, K), **u8)
        x8t = f8lin.new_transposed(K, M, dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        key = (weight.data_ptr(), weight._version, weight.dtype, str(dev), layer._mode("w"))
        cached = layer._w_cache if (layer.config.reuse_weight_cast and layer._w_cache is not None
                                    and layer._w_cache[0] == key) else None
        mode_x, sx = layer._prepare("x", x)
        if cached is not None:
            # unchanged weight: its fp8 copies and scale (in the w state) are still valid
            w, w8, w8t = None, cached[1], cached[2]
            mode_w, sw = "dynamic", layer.state("w")
            layer.weight_cast_reuses += 1
        else:
            # fresh copies: an earlier forward's backward may still read the old ones
            w = weight.to(torch.bfloat16).contiguous()
            w8 = torch.empty((N, K), **u8)
            w8t = f8lin.new_transposed(K, N, dev)
            mode_w, sw = layer._prepare("w", w)
        f8lin.forward(x, w, y, x8, x8t, w8, w8t, sx, sw, layer.fp8_workspace, mode_x, mode_w,
                      layer.config.amax_algo, bias=b, w_cast_valid=cached is not None)
        if cached is None and layer.config.reuse_weight_cast:
            layer._w_cache = (key, w8, w8t)
        # backward must use the scales these fp8 copies were made with, even if
        # the layer runs forward again before it (micro-batches, recomputation)
        ctx.save_for_backward(x8t, w8t, sx.scale.clone(), sw.scale.clone())
        ctx.layer = layer
        ctx.M0 = M0
        ctx.w_dtype = weight.dtype
        ctx.b_dtype = None if bias is None else bias.dtype
        return y[:M0]

    @staticmethod
    def backward(ctx, dy2d):
        x8t, w8t, sx_scale, sw_scale = ctx.saved_tensors
        layer = ctx.layer
        dy = _pad_rows(dy2d.to(torch.bfloat16))
        M, N = dy.shape
        K = x8t.shape[0]
        dev = dy.device
        dy8 = torch.empty((M, N), dtype=torch.uint8, device=dev)
        dy8t = f8lin.new_transposed(N, M, dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        db = db_ws = None
        if ctx.b_dtype is not None:
            db = torch.empty((N,), dtype=torch.bfloat16, device=dev)
            db_ws = f8lin.new_dbias_workspace(M, N, dev)
        # scratch for GEMMs split along their contraction (None when none splits at this shape)
        gemm_ws = f8lin.new_backward_gemm_workspace(M, N, K, dev)
        mode_dy, sdy = layer._prepare("dy", dy)
        f8lin.backward(dy, x8t, w8t, dx, dw, dy8, dy8t, f8lin.ScaleView(sx_scale), f8lin.ScaleView(sw_scale),
                       sdy, layer.fp8_workspace, mode_dy, layer.config.amax_algo, dbias=db, dbias_ws=db_ws,
                       gemm_ws=gemm_ws)
        return dx[:ctx.M0], dw.to(ctx.w_dtype), (None if db is None else db.to(ctx.b_dtype)), None


class Float8Linear(nn.Module):
    """nn.Linear whose forward and backward GEMMs run in fp8 with tensorwise
    scaling: X and W cast to e4m3, dY to e5m2, per-tensor scales from the
    current amax (dynamic) or a 16-step amax history (delayed)."""

    def __init__(self, in_features: int, out_features: int, config: Optional[Float8LinearConfig] = None,
                 weight: Optional[torch.Tensor] = None, device=None, dtype=torch.bfloat16, bias=False):
        super().__init__()
        if in_features % 16 or out_features % 16:
            raise ValueError("Float8Linear needs in_features and out_features that are multiples of 16")
        self.in_features = in_features
        self.out_features = out_features
        self.config = config or Float8LinearConfig()
        if weight is None:
            weight = torch.empty((out_features, in_features), device=device, dtype=dtype)
            nn.init.kaiming_uniform_(weight, a=5 ** 0.5)
        self.weight = weight if isinstance(weight, nn.Parameter) else nn.Parameter(weight)
        # bias: False / True (a zero-initialised bias), or an existing tensor / Parameter to share
        if isinstance(bias, torch.Tensor):
            if tuple(bias.shape) != (out_features,):
                raise ValueError("bias must have shape (out_features,)")
            self.bias = bias if isinstance(bias, nn.Parameter) else nn.Parameter(bias)
        elif bias:
            self.bias = nn.Parameter(torch.zeros(out_features, device=self.weight.device, dtype=self.weight.dtype))
        else:
            self.register_parameter("bias", None)
        dev = self.weight.device
        for role in _ROLES:
            for name, shape, dt in _STATE_FIELDS:
                self.register_buffer(f"fp8_{role}_{name}", torch.zeros(shape, dtype=dt, device=dev))
        # the library's workspace, and one history per role whose slot 0 holds
        # the current amax during a delayed role's first step (slots 1-15 stay 0)
        self.register_buffer("fp8_workspace", torch.zeros(f8lin.workspace_bytes(), dtype=torch.uint8, device=dev),
                             persistent=False)
        self.register_buffer("fp8_seed_history", torch.zeros((len(_ROLES), f8lin.HISTORY_LEN), dtype=torch.float32,
                                                             device=dev), persistent=False)
        self._initialized: Dict[str, bool] = {r: False for r in _ROLES}
        self._produced: Dict[str, bool] = {r: False for r in _ROLES}
        self._w_cache = None  # (key, w8, w8t) of the weight's last cast
        self.weight_cast_reuses = 0

    # ---- scaling state
    def state(self, role: str) -> f8lin.ScalingState:
        """The role's device state (views of this module's buffers)."""
        return f8lin.ScalingState(tensors=tuple(getattr(self, f"fp8_{role}_{n}") for n, _, _ in _STATE_FIELDS))

    sx = property(lambda self: self.state("x"))
    sw = property(lambda self: self.state("w"))
    sdy = property(lambda self: self.state("dy"))

    def _cfg(self, role):
        return {"x": self.config.cast_config_input, "w": self.config.cast_config_weight,
                "dy": self.config.cast_config_grad_output}[role]

    def _mode(self, role):
        """How the role's scale is taken this step: "delayed" (from the
        history) once the role has been synced, else "dynamic" (the current
        tensor's amax; for a delayed role this is its first step)."""
        if self._cfg(role).scaling_type == "delayed" and self._initialized[role]:
            return "delayed"
        return "dynamic"

    def _prepare(self, role, t: torch.Tensor):
        """(mode, state) for casting tensor t of `role`, and marks the role as
        having produced an amax since the last sync."""
        self._produced[role] = True
        st = self.state(role)
        if self._cfg(role).scaling_type == "dynamic" or self._initialized[role]:
            return self._mode(role), st
        # a delayed role's first step: the delayed cast with a history seeded
        # with this tensor's amax (the dynamic scale; the cast folds the amax
        # into the state, max over micro-batches)
        seed = self.fp8_seed_history[_ROLES.index(role)]
        f8lin.amax(t, seed[0:1], self.fp8_workspace, self.config.amax_algo)
        return "delayed", f8lin.ScalingState(tensors=(st.amax, st.scale, seed, st.hist_meta))

    def delayed_states(self):
        """States of the delayed roles that produced an amax since the last sync."""
        return [self.state(r) for r in self._sync_roles()]

    def _sync_roles(self):
        return [r for r in _ROLES if self._cfg(r).scaling_type == "delayed" and self._produced[r]]

    def _mark_synced(self, roles=None):
        for r in (self._sync_roles() if roles is None else roles):
            self._initialized[r] = True
            self._produced[r] = False
        self._w_cache = None  # the weight's scale may move with its history; the step is over

    def invalidate_weight_cast(self):
        """Drop the cached weight cast (after changing the weight through .data)."""
        self._w_cache = None

    # ---- checkpointing: the buffers are saved by nn.Module; the flags here
    def get_extra_state(self):
        return {"initialized": [bool(self._initialized[r]) for r in _ROLES]}

    def set_extra_state(self, state):
        flags = state["initialized"]
        self._initialized = {r: bool(f) for r, f in zip(_ROLES, flags)}
        self._produced = {r: False for r in _ROLES}
        self._w_cache = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not x.is_cuda:
            raise RuntimeError("Float8Linear runs on the GPU only (libf8lin has no CPU path)")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        if self.fp8_x_amax.device != x.device:
            raise RuntimeError(f"Float8Linear's scaling state is on {self.fp8_x_amax.device}, the input on "
                               f"{x.device}: move the module with .to()")
        lead = x.shape[:-1]
        y = _Float8LinearFn.apply(x.reshape(-1, self.in_features), self.weight, self.bias, self)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        c = self.config
        return (f"in_features={self.in_features}, out_features={self.out_features}, bias={self.bias is not None}, "
                f"input={c.cast_config_input.scaling_type}, weight={c.cast_config_weight.scaling_type}, "
                f"grad_output={c.cast_config_grad_output.scaling_type}, amax_algo={c.amax_algo}")


def convert_to_float8_training(module: nn.Module, config: Optional[Float8LinearConfig] = None,
                               module_filter_fn=None) -> nn.Module:
    """Replaces every nn.Linear whose dimensions are multiples of 16 (and that
    module_filter_fn(fqn, module) accepts, if given) by a Float8Linear sharing
    its weight and bias Parameters.  Returns the module."""
    config = config or Float8LinearConfig()

    def swap(parent: nn.Module, prefix: str):
        for name, child in list(parent.named_children()):
            fqn = f"{prefix}.{name}" if prefix else name
            if (type(child) is nn.Linear and child.in_features % 16 == 0 and child.out_features % 16 == 0
                    and (module_filter_fn is None or module_filter_fn(fqn, child))):
                setattr(parent, name, Float8Linear(child.in_features, child.out_features, config,
                                                   weight=child.weight,
                                                   bias=child.bias if child.bias is not None else False))
            else:
                swap(child, fqn)

    if type(module) is nn.Linear:
        raise ValueError("convert the parent module, not a bare nn.Linear")
    swap(module, "")
    return module


def invalidate_weight_cast(module: nn.Module) -> None:
    """Drops every Float8Linear's cached weight cast (call it after changing
    weights through .data when reuse_weight_cast is on)."""
    for m in module.modules():
        if isinstance(m, Float8Linear):
            m.invalidate_weight_cast()


def sync_float8_amax_and_scale_history(module: nn.Module, check: bool = False) -> None:
    """After backward: pushes the amax of this step of every delayed-scaling
    role that produced one into its 16-entry history (one launch for all
    layers' states).  check=True also reads back the library's per-state
    status (a host synchronisation) and raises if a state's {count, pos}
    was corrupt (such a state is left untouched)."""
    states, layers = [], []
    for m in module.modules():
        if isinstance(m, Float8Linear):
            roles = m._sync_roles()
            states.extend(m.state(r) for r in roles)
            layers.append((m, roles))
    status = None
    if states:
        if check:
            status = torch.empty(len(states), dtype=torch.int32, device=states[0].amax.device)
        f8lin.delayed_update(states, status=status)
    for m, roles in layers:
        m._mark_synced(roles)
    if status is not None:
        bad = torch.nonzero(status).flatten().tolist()
        if bad:
            raise RuntimeError(f"sync_float8_amax_and_scale_history: {len(bad)} corrupt delayed-scaling "
                               f"state(s) (invalid count/pos), left unchanged: state indices {bad}")
