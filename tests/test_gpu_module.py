"""The PyTorch module surface (Float8Linear, convert_to_float8_training,
sync_float8_amax_and_scale_history) against the oracle: every number still
comes from libf8lin's kernels, reached through autograd."""
import numpy as np
import pytest
import torch
import torch.nn as nn

import oracle
from float8linear_tensorwise_amax_amd import inputs
from helpers import bf16_to_f64, bits, f32_bits, gemm_check, np_f32_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def mod():
    from float8linear_tensorwise_amax_amd import module
    return module


def _pad(a: np.ndarray, rows: int) -> np.ndarray:
    out = np.zeros((rows, a.shape[1]), dtype=a.dtype)
    out[:a.shape[0]] = a
    return out


def test_module_forward_backward_matches_oracle(mod):
    torch.manual_seed(0)
    layer = mod.Float8Linear(96, 160, weight=inputs.random_bf16((160, 96), seed=3, std=96 ** -0.5).to(DEV))
    x = inputs.random_bf16((3, 7, 96), seed=4).to(DEV).requires_grad_(True)  # 21 rows: padded to 32
    dy = inputs.random_bf16((3, 7, 160), seed=5, std=1e-3 ** 0.5).to(DEV)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xb = _pad(bits(x.detach().reshape(21, 96)), 32)
    dyb = _pad(bits(dy.reshape(21, 160)), 32)
    ref = oracle.linear_step(xb, bits(layer.weight.detach()), dyb)
    assert f32_bits(layer.sx.amax)[0] == np_f32_bits(ref["x"]["amax"])
    assert f32_bits(layer.sdy.scale)[0] == np_f32_bits(ref["dy"]["scale"])
    gemm_check(bf16_to_f64(y.detach().reshape(21, 160)), ref["y"][:21], rms=float(np.sqrt(np.mean(ref["y"] ** 2))),
               what="module Y")
    gemm_check(bf16_to_f64(x.grad.reshape(21, 96)), ref["dx"][:21], rms=float(np.sqrt(np.mean(ref["dx"] ** 2))),
               what="module dX")
    gemm_check(bf16_to_f64(layer.weight.grad), ref["dw"], what="module dW")


def test_convert_and_delayed_sync(mod):
    torch.manual_seed(1)
    model = nn.Sequential(nn.Linear(64, 128, bias=False), nn.GELU(), nn.Linear(128, 64, bias=False)).to(DEV)
    model = model.to(torch.bfloat16)
    cfg = mod.Float8LinearConfig(cast_config_input=mod.CastConfig("delayed"),
                                 cast_config_weight=mod.CastConfig("delayed"),
                                 cast_config_grad_output=mod.CastConfig("delayed"))
    mod.convert_to_float8_training(model, cfg)
    assert isinstance(model[0], mod.Float8Linear) and isinstance(model[2], mod.Float8Linear)
    hist = oracle.DelayedHistory()
    for step in range(4):
        x = inputs.random_bf16((48, 64), seed=10 + step, std=1.0 + step).to(DEV)
        assert model[0]._mode("x") == ("dynamic" if step == 0 else "delayed")
        y = model(x)
        y.float().sum().backward()
        mod.sync_float8_amax_and_scale_history(model)
        torch.cuda.synchronize()
        xb = bits(x)
        s_expect, _ = oracle.scale(hist.amax_for_scale(xb), oracle.E4M3)
        assert f32_bits(model[0].sx.scale)[0] == np_f32_bits(s_expect), step
        hist.push(oracle.amax(xb))
        assert np.array_equal(f32_bits(model[0].sx.history), hist.hist.view(np.uint32)), step
        for p in model.parameters():
            p.grad = None


def test_forward_twice_before_backward_uses_saved_scales(mod):
    """Two micro-batches through one layer before backward: each backward
    uses the scales its own forward cast with."""
    layer = mod.Float8Linear(64, 32, weight=inputs.random_bf16((32, 64), seed=7, std=0.125).to(DEV))
    xa = inputs.random_bf16((16, 64), seed=8, std=1.0).to(DEV).requires_grad_(True)
    xb_ = inputs.random_bf16((16, 64), seed=9, std=50.0).to(DEV).requires_grad_(True)
    dy = inputs.random_bf16((16, 32), seed=11, std=0.03).to(DEV)
    ya = layer(xa)
    yb = layer(xb_)
    ya.backward(dy)
    ga = layer.weight.grad.clone()
    layer.weight.grad = None
    yb.backward(dy)
    torch.cuda.synchronize()
    ref = oracle.linear_step(bits(xa.detach()), bits(layer.weight.detach()), bits(dy))
    gemm_check(bf16_to_f64(ga), ref["dw"], what="micro-batch A dW")
    gemm_check(bf16_to_f64(xa.grad), ref["dx"], what="micro-batch A dX")


def test_module_with_bias_matches_oracle(mod):
    """A biased layer (the repro's nn.Linear layers keep their bias): Y
    includes b, and bias.grad is the column sum of dY."""
    from helpers import bf16_ulp
    w = inputs.random_bf16((160, 96), seed=13, std=96 ** -0.5).to(DEV)
    b = inputs.random_bf16((160,), seed=14, std=0.2).to(DEV)
    layer = mod.Float8Linear(96, 160, weight=w, bias=b.clone())
    x = inputs.random_bf16((3, 7, 96), seed=15).to(DEV).requires_grad_(True)  # 21 rows: padded to 32
    dy = inputs.random_bf16((3, 7, 160), seed=16, std=1e-3 ** 0.5).to(DEV)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xb = _pad(bits(x.detach().reshape(21, 96)), 32)
    dyb = _pad(bits(dy.reshape(21, 160)), 32)
    ref = oracle.linear_step(xb, bits(layer.weight.detach()), dyb, bias_bits=bits(layer.bias.detach()))
    gemm_check(bf16_to_f64(y.detach().reshape(21, 160)), ref["y"][:21], rms=float(np.sqrt(np.mean(ref["y"] ** 2))),
               what="module Y + b")
    got = bf16_to_f64(layer.bias.grad)
    absum = np.abs(oracle.bf16_to_f64(dyb)).sum(axis=0)
    assert np.all(np.abs(got - ref["dbias"]) <= 1e-5 * absum + bf16_ulp(ref["dbias"]))


def test_module_reuses_the_weight_cast_between_micro_batches(mod):
    """Micro-batches before an optimizer step reuse the weight's fp8 copies
    (same bits as recasting); an in-place update of the weight recasts it."""
    torch.manual_seed(3)
    w = inputs.random_bf16((128, 64), seed=31, std=0.125).to(DEV)
    layer = mod.Float8Linear(64, 128, weight=w.clone())
    fresh = mod.Float8Linear(64, 128, weight=w.clone(), config=mod.Float8LinearConfig(reuse_weight_cast=False))
    xs = [inputs.random_bf16((32, 64), seed=32 + i).to(DEV) for i in range(3)]
    dy = inputs.random_bf16((32, 128), seed=40, std=0.03).to(DEV)
    for i, x in enumerate(xs):
        y = layer(x)
        y.backward(dy)
        y2 = fresh(x)
        y2.backward(dy)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), i
    assert layer.weight_cast_reuses == 2 and fresh.weight_cast_reuses == 0
    assert torch.equal(layer.weight.grad.view(torch.int16), fresh.weight.grad.view(torch.int16))
    with torch.no_grad():
        layer.weight.mul_(2.0)  # in place: the version counter moves
        fresh.weight.mul_(2.0)
    y, y2 = layer(xs[0]), fresh(xs[0])
    torch.cuda.synchronize()
    assert layer.weight_cast_reuses == 2
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
