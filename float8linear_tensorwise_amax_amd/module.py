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
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch
import torch.nn as nn

from . import f8lin


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
    # Reuse the weight's fp8 copies while the weight is unchanged (same tensor,
    # same version counter: e.g. the micro-batches of one optimizer step).
    reuse_weight_cast: bool = True


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
        w = weight.to(torch.bfloat16).contiguous()
        b = None if bias is None else bias.to(torch.bfloat16).contiguous()
        M, K = x.shape
        N = w.shape[0]
        dev = x.device
        u8 = dict(dtype=torch.uint8, device=dev)
        x8 = torch.empty((M, K), **u8)
        x8t = torch.empty((K, M), **u8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        mode_x = layer._mode("x")
        mode_w = layer._mode("w")
        key = (weight.data_ptr(), weight._version, weight.dtype, str(dev), mode_w)
        cached = layer._w_cache if (layer.config.reuse_weight_cast and layer._w_cache is not None
                                    and layer._w_cache[0] == key) else None
        if cached is not None:
            # unchanged weight: its fp8 copies and scale (in layer.sw) are still valid
            w8, w8t = cached[1], cached[2]
            layer.weight_cast_reuses += 1
        else:
            # fresh copies: an earlier forward's backward may still read the old ones
            w8 = torch.empty((N, K), **u8)
            w8t = torch.empty((K, N), **u8)
        f8lin.forward(x, None if cached is not None else w, y, x8, x8t, w8, w8t, layer.sx, layer.sw, layer.ws,
                      mode_x, mode_w, layer.config.amax_algo, bias=b, w_cast_valid=cached is not None)
        if cached is None and layer.config.reuse_weight_cast:
            layer._w_cache = (key, w8, w8t)
        # backward must use the scales these fp8 copies were made with, even if
        # the layer runs forward again before it (micro-batches, recomputation)
        ctx.save_for_backward(x8t, w8t, layer.sx.scale.clone(), layer.sw.scale.clone())
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
        dy8t = torch.empty((N, M), dtype=torch.uint8, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        db = db_ws = None
        if ctx.b_dtype is not None:
            db = torch.empty((N,), dtype=torch.bfloat16, device=dev)
            db_ws = f8lin.new_dbias_workspace(M, N, dev)
        # scratch for GEMMs split along their contraction (None when none splits at this shape)
        gemm_ws = f8lin.new_backward_gemm_workspace(M, N, K, dev)
        f8lin.backward(dy, x8t, w8t, dx, dw, dy8, dy8t, f8lin.ScaleView(sx_scale), f8lin.ScaleView(sw_scale),
                       layer.sdy, layer.ws, layer._mode("dy"), layer.config.amax_algo, dbias=db, dbias_ws=db_ws,
                       gemm_ws=gemm_ws)
        return dx[:ctx.M0], dw.to(ctx.w_dtype), (None if db is None else db.to(ctx.b_dtype)), None


class Float8Linear(nn.Module):
    """nn.Linear (no bias) whose forward and backward GEMMs run in fp8 with
    tensorwise scaling: X and W cast to e4m3, dY to e5m2, per-tensor scales
    from the current amax (dynamic) or a 16-step amax history (delayed)."""

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
        self._states_device = None
        self._initialized: Dict[str, bool] = {"x": False, "w": False, "dy": False}
        self._w_cache = None  # (key, w8, w8t) of the weight's last cast
        self.weight_cast_reuses = 0

    # ---- scaling state (device-resident, created on first use on the weight's device)
    def _ensure_states(self, device):
        if self._states_device != device:
            self.sx = f8lin.ScalingState(device)
            self.sw = f8lin.ScalingState(device)
            self.sdy = f8lin.ScalingState(device)
            self.ws = f8lin.new_workspace(device)
            self._states_device = device
            self._initialized = {"x": False, "w": False, "dy": False}
            self._w_cache = None

    def _cfg(self, role):
        return {"x": self.config.cast_config_input, "w": self.config.cast_config_weight,
                "dy": self.config.cast_config_grad_output}[role]

    def _mode(self, role):
        # delayed scaling takes its first step's scale from the current amax
        if self._cfg(role).scaling_type == "delayed" and self._initialized[role]:
            return "delayed"
        return "dynamic"

    def delayed_states(self):
        return [st for role, st in (("x", getattr(self, "sx", None)), ("w", getattr(self, "sw", None)),
                                    ("dy", getattr(self, "sdy", None)))
                if st is not None and self._cfg(role).scaling_type == "delayed"]

    def _mark_synced(self):
        for role in ("x", "w", "dy"):
            if self._cfg(role).scaling_type == "delayed":
                self._initialized[role] = True
        if self._cfg("w").scaling_type == "delayed":
            self._w_cache = None  # the history moved: the weight's scale changes

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not x.is_cuda:
            raise RuntimeError("Float8Linear runs on the GPU only (libf8lin has no CPU path)")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        self._ensure_states(x.device)
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


def sync_float8_amax_and_scale_history(module: nn.Module) -> None:
    """After backward: pushes every delayed-scaling tensor's amax of this
    step into its 16-entry history (one launch for all layers' states)."""
    states = []
    layers = []
    for m in module.modules():
        if isinstance(m, Float8Linear) and m._states_device is not None:
            states.extend(m.delayed_states())
            layers.append(m)
    if states:
        f8lin.delayed_update(states)
    for m in layers:
        m._mark_synced()
