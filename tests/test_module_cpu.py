"""Host-side logic of the module surface: which layers are swapped, config
validation and scaling-mode bookkeeping (no GPU work)."""
import pytest
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
    cfg = m.Float8LinearConfig(cast_config_weight=m.CastConfig("delayed"))
    layer = m.Float8Linear(32, 48, cfg)
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["dynamic"] * 3  # first step: amax init
    layer._mark_synced()
    assert [layer._mode(r) for r in ("x", "w", "dy")] == ["dynamic", "delayed", "dynamic"]
    with pytest.raises(ValueError):
        m.Float8Linear(30, 48)
