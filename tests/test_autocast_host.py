"""Host logic of the fp8 policy layer (no GPU): formats, recipe checks,
fp8_autocast regions (nesting, threads), the disabled path and the
per-weight state."""

import gc
import threading

import pytest
import torch

from fp8_tensor_scaled_amd import E4M3, E5M2
from fp8_tensor_scaled_amd import autocast as fa


def test_formats():
    assert (fa.FP8Format.HYBRID.fwd(), fa.FP8Format.HYBRID.bwd()) == (E4M3, E5M2)
    assert (fa.FP8Format.E4M3.fwd(), fa.FP8Format.E4M3.bwd()) == (E4M3, E4M3)
    assert (fa.FP8Format.E5M2.fwd(), fa.FP8Format.E5M2.bwd()) == (E5M2, E5M2)
    assert fa.FP8Format("hybrid") is fa.FP8Format.HYBRID


@pytest.mark.parametrize("kw", [dict(history_len=0), dict(history_len=5000), dict(margin=-1),
                                dict(margin=65)])
def test_recipe_rejects_bad_values(kw):
    with pytest.raises(ValueError):
        fa.FP8Recipe(**kw)


def test_autocast_regions_nest_and_restore():
    fa.fp8_state().reset()
    assert not fa.current_config().enabled
    r1, r2 = fa.FP8Recipe(history_len=4), fa.FP8Recipe(dynamic=True, margin=2)
    with fa.fp8_autocast(recipe=r1):
        c = fa.current_config()
        assert c.enabled and c.recipe == r1 and c.fp8_format is fa.FP8Format.HYBRID
        with fa.fp8_autocast(enabled=False):
            assert not fa.current_config().enabled
            with fa.fp8_autocast(recipe=r2, fp8_format="e4m3"):
                c = fa.current_config()
                assert c.recipe == r2 and c.fp8_format is fa.FP8Format.E4M3
            assert not fa.current_config().enabled
        assert fa.current_config().recipe == r1
    assert not fa.current_config().enabled


def test_autocast_is_per_thread():
    seen = {}

    def other():
        seen["enabled"] = fa.current_config().enabled

    with fa.fp8_autocast():
        t = threading.Thread(target=other)
        t.start()
        t.join()
        assert fa.current_config().enabled
    assert seen["enabled"] is False


def test_defaults_and_reset():
    st = fa.fp8_state()
    st.default_enabled = True
    st.default_recipe = fa.FP8Recipe(history_len=8)
    assert fa.current_config().enabled and fa.current_config().recipe.history_len == 8
    st.reset()
    assert not fa.current_config().enabled and fa.current_config().recipe == fa.FP8Recipe()


def test_disabled_path_is_plain_linear():
    fa.fp8_state().reset()
    x = torch.randn(3, 5, 8)
    w = torch.randn(4, 8)
    b = torch.randn(4)
    assert torch.equal(fa.fp8_linear(x, w, b), torch.nn.functional.linear(x, w, b))
    with fa.fp8_autocast(enabled=False):
        m = fa.FP8Linear(8, 4)
        assert torch.equal(m(x), torch.nn.functional.linear(x, m.weight, m.bias))


def test_enabled_path_checks_dtypes():
    with fa.fp8_autocast():
        with pytest.raises(ValueError, match="bfloat16"):
            fa.fp8_linear(torch.randn(2, 8), torch.randn(4, 8).bfloat16())
        with pytest.raises(ValueError, match="w_scale"):
            fa.fp8_linear(torch.randn(2, 8).bfloat16(), torch.zeros(4, 8).to(torch.float8_e4m3fn))


def test_enabled_path_checks_shapes():
    """The shapes are checked before anything reaches the library: the
    input's last dimension against the weight's, the bias against the
    weight's outputs."""
    with fa.fp8_autocast():
        with pytest.raises(ValueError, match="do not match"):
            fa.fp8_linear(torch.randn(2, 6).bfloat16(), torch.randn(4, 8).bfloat16())
        with pytest.raises(ValueError, match="bias of shape"):
            fa.fp8_linear(torch.randn(2, 8).bfloat16(), torch.randn(4, 8).bfloat16(),
                          torch.randn(3).bfloat16())


def test_weight_meta_lifetime():
    st = fa.fp8_state()
    st.reset()
    w = torch.zeros(4, 8)
    r = fa.FP8Recipe(history_len=4)
    m1 = st.get_weight_meta(w, r)
    assert st.get_weight_meta(w, r) is m1
    assert m1.x.len == 4 and m1.g.idx == 0 and not m1.w.initialized
    assert st.get_weight_meta(w, fa.FP8Recipe(history_len=8)) is not m1  # new window length
    n = len(st._metas)
    del w
    gc.collect()
    assert len(st._metas) == n - 1


def test_linear_routing_switch_host():
    """fp8_linear_enable registers and removes the aten::linear kernels of
    CUDA tensors; CPU calls never change."""
    x, lin = torch.randn(4, 8), torch.nn.Linear(8, 3)
    want = lin(x)
    fa.fp8_linear_enable(True)
    try:
        assert fa.fp8_linear_enabled()
        fa.fp8_linear_enable(True)  # idempotent
        with fa.fp8_autocast():
            assert torch.equal(lin(x), want)
    finally:
        fa.fp8_linear_enable(False)
    assert not fa.fp8_linear_enabled()
    fa.fp8_linear_enable(False)
    assert torch.equal(lin(x), want)
