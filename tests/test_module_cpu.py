"""Host-side logic of the module surface: which layers are swapped, config
validation and scaling-mode bookkeeping (no GPU work)."""
import pytest
import torch
import torch.nn as nn

from float8linear_tensorwise_amax_amd import module as m


def test_convert_swaps_only_eligible_linears():
    model = nn.Sequential(nn.Linear(64, 128, bias=False), nn.ReLU(), nn.Linear(128, 60, bias=False),
                          nn.Linear(60, 64, bias=True), nn.Sequential(nn.Linear(32, 32, bias=False)))
    w0 = model[0].weight
    m.convert_to_float8_training(model)
    assert isinstance(model[0], m.Float8Linear) and model[0].weight is w0  # weight shared, not copied
    assert type(model[2]) is nn.Linear  # out_features not a multiple of 16
    assert type(model[3]) is nn.Linear  # in_features not a multiple of 16
    assert isinstance(model[4][0], m.Float8Linear)
    model = nn.Sequential(nn.Linear(64, 128, bias=True))
    b0 = model[0].bias
    m.convert_to_float8_training(model)
    assert isinstance(model[0], m.Float8Linear) and model[0].bias is b0  # bias shared too


def test_convert_with_filter_and_bare_linear():
    model = nn.Sequential(nn.Linear(32, 32, bias=False), nn.Linear(32, 32, bias=False))
    m.convert_to_float8_training(model, module_filter_fn=lambda fqn, mod: fqn != "1")
    assert isinstance(model[0], m.Float8Linear) and type(model[1]) is nn.Linear
    with pytest.raises(ValueError):
        m.convert_to_float8_training(nn.Linear(32, 32, bias=False))


def test_config_validation_and_modes():
    with pytest.raises(ValueError):
        m.CastConfig("rowwise")
    cfg = m.Float8LinearConfig(cast_config_weight=m.CastConfig("delayed"), cast_config_grad_output=m.CastConfig("delayed"))
    layer = m.Float8Linear(32, 48, cfg)
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["dynamic"] * 3  # first step: amax init
    # a sync with nothing produced since the last one initialises nothing
    layer._mark_synced()
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["dynamic"] * 3
    # a forward without backward produced the weight's amax, not grad_output's
    layer._produced["x"] = layer._produced["w"] = True
    assert layer._sync_roles() == ["w"]  # only delayed roles are pushed
    layer._mark_synced()
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["dynamic", "delayed", "dynamic"]
    assert layer._sync_roles() == []
    with pytest.raises(ValueError):
        m.Float8Linear(30, 48)


def test_weight_cast_reuse_is_opt_in():
    assert m.Float8LinearConfig().reuse_weight_cast is False
    layer = m.Float8Linear(32, 48, m.Float8LinearConfig(reuse_weight_cast=True))
    layer._w_cache = ("key", None, None)
    m.invalidate_weight_cast(nn.Sequential(layer))
    assert layer._w_cache is None
    layer._w_cache = ("key", None, None)
    layer._mark_synced()  # the sync ends the step: the cache goes too
    assert layer._w_cache is None


def test_scaling_state_is_in_the_state_dict():
    """amax, scale, history and {count, pos} of every role are buffers, and
    which delayed roles are initialised is the module's extra state: a
    save / load round trip restores both (the workspace is not saved)."""
    cfg = m.Float8LinearConfig(cast_config_input=m.CastConfig("delayed"))
    a = m.Float8Linear(32, 48, cfg, bias=True)
    sd = a.state_dict()
    for role in ("x", "w", "dy"):
        for f in ("amax", "scale", "history", "hist_meta"):
            assert f"fp8_{role}_{f}" in sd
    assert "fp8_workspace" not in sd and "fp8_seed_history" not in sd
    a.fp8_x_history[3] = 7.5
    a.fp8_x_hist_meta[:] = torch.tensor([4, 4], dtype=torch.int32)
    a._initialized["x"] = True
    b = m.Float8Linear(32, 48, cfg, bias=True)
    b.load_state_dict(a.state_dict())
    assert torch.equal(b.fp8_x_history, a.fp8_x_history) and torch.equal(b.fp8_x_hist_meta, a.fp8_x_hist_meta)
    assert b._mode("x") == "delayed" and b._mode("w") == "dynamic"
    assert b.sx.history.data_ptr() == b.fp8_x_history.data_ptr()  # the library reads the buffers themselves
