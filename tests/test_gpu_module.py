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
    layer = mod.Float8Linear(64, 128, weight=w.clone(), config=mod.Float8LinearConfig(reuse_weight_cast=True))
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


def test_weight_changed_through_data_is_recast(mod):
    """p.data.copy_ does not move the version counter.  Without reuse (the
    default) the forward always recasts; with reuse, invalidate_weight_cast
    makes it recast.  Both give the bits of a fresh layer."""
    w = inputs.random_bf16((128, 64), seed=51, std=0.125).to(DEV)
    w2 = inputs.random_bf16((128, 64), seed=52, std=0.5).to(DEV)
    x = inputs.random_bf16((32, 64), seed=53).to(DEV)
    default = mod.Float8Linear(64, 128, weight=w.clone())
    reuse = mod.Float8Linear(64, 128, weight=w.clone(), config=mod.Float8LinearConfig(reuse_weight_cast=True))
    ref = mod.Float8Linear(64, 128, weight=w2.clone())
    for layer in (default, reuse):
        with torch.no_grad():
            layer(x)
            layer.weight.data.copy_(w2)
    mod.invalidate_weight_cast(reuse)
    with torch.no_grad():
        outs = [default(x), reuse(x), ref(x)]
    torch.cuda.synchronize()
    assert reuse.weight_cast_reuses == 0
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    assert torch.equal(outs[1].view(torch.int16), outs[2].view(torch.int16))


def _delayed_model(mod, seed, bias=False):
    gen = torch.Generator().manual_seed(seed)
    model = nn.Sequential(nn.Linear(64, 96, bias=bias), nn.GELU(), nn.Linear(96, 48, bias=bias))
    with torch.no_grad():
        for p in model.parameters():
            p.copy_(torch.randn(p.shape, generator=gen) * 0.1)
    model = model.to(DEV).to(torch.bfloat16)
    cfg = mod.Float8LinearConfig(cast_config_input=mod.CastConfig("delayed"),
                                 cast_config_weight=mod.CastConfig("delayed"),
                                 cast_config_grad_output=mod.CastConfig("delayed"))
    return mod.convert_to_float8_training(model, cfg)


def test_step0_micro_batches_fold_their_amax(mod):
    """Two micro-batches at a delayed role's first step: each is cast with
    its own (dynamic) scale, and the sync pushes the max of their amaxes --
    as later steps fold theirs.  Checked against the oracle's history."""
    layer = mod.Float8Linear(64, 32, weight=inputs.random_bf16((32, 64), seed=61, std=0.125).to(DEV),
                             config=mod.Float8LinearConfig(cast_config_input=mod.CastConfig("delayed"),
                                                           cast_config_grad_output=mod.CastConfig("delayed")))
    xs = [inputs.random_bf16((16, 64), seed=62 + i, std=s).to(DEV) for i, s in enumerate((8.0, 1.0))]
    dys = [inputs.random_bf16((16, 32), seed=64 + i, std=s).to(DEV) for i, s in enumerate((0.01, 0.3))]
    hx, hdy = oracle.DelayedHistory(), oracle.DelayedHistory()
    for x, dy in zip(xs, dys):
        y = layer(x)
        y.backward(dy)
        torch.cuda.synchronize()
        # this micro-batch's cast used its own tensor's amax
        assert f32_bits(layer.sx.scale)[0] == np_f32_bits(oracle.scale(oracle.amax(bits(x)), oracle.E4M3)[0])
        assert f32_bits(layer.sdy.scale)[0] == np_f32_bits(oracle.scale(oracle.amax(bits(dy)), oracle.E5M2)[0])
    mod.sync_float8_amax_and_scale_history(layer, check=True)
    torch.cuda.synchronize()
    hx.push(max(oracle.amax(bits(xs[0])), oracle.amax(bits(xs[1]))))
    hdy.push(max(oracle.amax(bits(dys[0])), oracle.amax(bits(dys[1]))))
    assert np.array_equal(f32_bits(layer.sx.history), hx.hist.view(np.uint32))
    assert np.array_equal(f32_bits(layer.sdy.history), hdy.hist.view(np.uint32))
    assert tuple(layer.sx.hist_meta.cpu().tolist()) == (hx.count, hx.pos) == (1, 1)
    # the next step takes its scale from that history
    x = inputs.random_bf16((16, 64), seed=70).to(DEV)
    layer(x).backward(dys[0])
    torch.cuda.synchronize()
    assert f32_bits(layer.sx.scale)[0] == np_f32_bits(oracle.scale(hx.amax_for_scale(bits(x)), oracle.E4M3)[0])
    assert f32_bits(layer.sdy.scale)[0] == np_f32_bits(oracle.scale(hdy.amax_for_scale(bits(dys[0])),
                                                                    oracle.E5M2)[0])


def test_forward_only_step_pushes_no_grad_output_amax(mod):
    """A step whose forward ran without backward produces no grad_output
    amax: the sync pushes x and w only, grad_output stays uninitialised and
    its next step is an amax-initialisation step again."""
    layer = mod.Float8Linear(64, 32, weight=inputs.random_bf16((32, 64), seed=71, std=0.125).to(DEV),
                             config=mod.Float8LinearConfig(cast_config_input=mod.CastConfig("delayed"),
                                                           cast_config_weight=mod.CastConfig("delayed"),
                                                           cast_config_grad_output=mod.CastConfig("delayed")))
    x0 = inputs.random_bf16((16, 64), seed=72, std=3.0).to(DEV)
    with torch.no_grad():
        layer(x0)
    mod.sync_float8_amax_and_scale_history(layer, check=True)
    torch.cuda.synchronize()
    assert layer.sx.hist_meta.cpu().tolist() == [1, 1] and layer.sw.hist_meta.cpu().tolist() == [1, 1]
    assert layer.sdy.hist_meta.cpu().tolist() == [0, 0] and float(layer.sdy.history.abs().sum()) == 0.0
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["delayed", "delayed", "dynamic"]
    hx = oracle.DelayedHistory()
    hx.push(oracle.amax(bits(x0)))
    x1 = inputs.random_bf16((16, 64), seed=73).to(DEV)
    dy1 = inputs.random_bf16((16, 32), seed=74, std=0.05).to(DEV)
    layer(x1).backward(dy1)
    torch.cuda.synchronize()
    assert f32_bits(layer.sx.scale)[0] == np_f32_bits(oracle.scale(hx.amax_for_scale(bits(x1)), oracle.E4M3)[0])
    assert f32_bits(layer.sdy.scale)[0] == np_f32_bits(oracle.scale(oracle.amax(bits(dy1)), oracle.E5M2)[0])


def test_module_checkpoint_resume_equals_uninterrupted(mod):
    """A two-layer model with delayed scaling of every role, 20 steps of fresh
    inputs (the GPT block's schedule at a small size): save model.state_dict()
    at step 10, load it into a new model, continue -- every output, gradient
    and scaling state equals the uninterrupted run's, bit for bit."""
    def steps(model, t0, t1):
        outs = []
        for t in range(t0, t1):
            x = inputs.random_bf16((40, 64), seed=500 + t, std=1.0 + (t % 5)).to(DEV)
            y = model(x)
            y.float().square().sum().backward()
            mod.sync_float8_amax_and_scale_history(model, check=True)
            outs.append((y.detach().clone(), [p.grad.clone() for p in model.parameters()]))
            for p in model.parameters():
                p.grad = None
        torch.cuda.synchronize()
        return outs

    a = _delayed_model(mod, 5, bias=True)
    full = steps(a, 0, 20)
    b = _delayed_model(mod, 5, bias=True)
    steps(b, 0, 10)
    saved = {k: v.detach().cpu().clone() if isinstance(v, torch.Tensor) else v for k, v in b.state_dict().items()}
    c = _delayed_model(mod, 5, bias=True)
    c.load_state_dict(saved)
    rest = steps(c, 10, 20)
    for (ya, ga), (yc, gc) in zip(full[10:], rest):
        assert torch.equal(ya.view(torch.int16), yc.view(torch.int16))
        for p, q in zip(ga, gc):
            assert torch.equal(p.view(torch.int16), q.view(torch.int16))
    for k, v in a.state_dict().items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(v, c.state_dict()[k]), k


def test_corrupt_delayed_state_is_reported_and_left_untouched(mod):
    """A state whose {count, pos} no sequence of pushes can reach (count > 16,
    pos out of range, or pos != count before the ring is full) is invalid
    data, not a fault: the update leaves it as it is and reports it in the
    status array; valid states in the same call are updated."""
    from float8linear_tensorwise_amax_amd import f8lin
    good = f8lin.ScalingState(DEV)
    good.amax.fill_(2.5)
    bad = []
    for meta in ([17, 0], [3, 16], [-1, 0], [5, 2], [16, -1]):
        st = f8lin.ScalingState(DEV)
        st.amax.fill_(9.0)
        st.history.copy_(torch.arange(16, dtype=torch.float32))
        st.hist_meta.copy_(torch.tensor(meta, dtype=torch.int32))
        bad.append(st)
    full = f8lin.ScalingState(DEV)  # a full ring at any position is valid
    full.hist_meta.copy_(torch.tensor([16, 7], dtype=torch.int32))
    full.amax.fill_(1.25)
    states = [good] + bad + [full]
    before = [(s.amax.clone(), s.history.clone(), s.hist_meta.clone()) for s in bad]
    status = torch.full((len(states),), 99, dtype=torch.int32, device=DEV)
    f8lin.delayed_update(states, status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 1, 1, 1, 1, 1, 0]
    for s, (a0, h0, m0) in zip(bad, before):
        assert torch.equal(s.amax, a0) and torch.equal(s.history, h0) and torch.equal(s.hist_meta, m0)
    assert good.hist_meta.cpu().tolist() == [1, 1] and float(good.history[0]) == 2.5 and float(good.amax) == 0.0
    assert full.hist_meta.cpu().tolist() == [16, 8] and float(full.history[7]) == 1.25
    # without a status array the invalid states are still left alone
    f8lin.delayed_update(bad)
    torch.cuda.synchronize()
    for s, (a0, h0, m0) in zip(bad, before):
        assert torch.equal(s.amax, a0) and torch.equal(s.history, h0) and torch.equal(s.hist_meta, m0)
    # the module's sync raises on them when asked to check
    layer = mod.Float8Linear(32, 16, weight=inputs.random_bf16((16, 32), seed=81).to(DEV),
                             config=mod.Float8LinearConfig(cast_config_input=mod.CastConfig("delayed")))
    with torch.no_grad():
        layer(inputs.random_bf16((16, 32), seed=82).to(DEV))
    layer.fp8_x_hist_meta.copy_(torch.tensor([20, 3], dtype=torch.int32))
    with pytest.raises(RuntimeError, match="corrupt"):
        mod.sync_float8_amax_and_scale_history(layer, check=True)
