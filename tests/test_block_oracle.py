"""The block oracle against its pins, and plausible mistakes planted in copies of
it (each must fail at least one pin). CPU only."""
import importlib.util
import os
import sys

import pytest

import oracle
import oracle.block
import pins_block


@pytest.mark.parametrize("pin", pins_block.BLOCK_PINS, ids=lambda f: f.__name__)
def test_block_pin(pin):
    pin(oracle.block)


MUTANTS = {
    "x_and_z_halves_swapped": [("xi, z = proj[..., :Din], proj[..., Din:]", "z, xi = proj[..., :Din], proj[..., Din:]")],
    "no_residual": [("out = x + y @ np.asarray(W[\"W_out\"], np.float64).T", "out = y @ np.asarray(W[\"W_out\"], np.float64).T")],
    "norm_without_scale": [("* np.asarray(w, np.float64)", "* 1.0")],
    "norm_mean_not_rms": [("np.mean(x * x, axis=-1, keepdims=True)", "np.mean(np.abs(x), axis=-1, keepdims=True) ** 2")],
    "b_and_c_swapped": [("dr, Bm, Cm = xp[..., :R], xp[..., R:R + N], xp[..., R + N:]",
                         "dr, Cm, Bm = xp[..., :R], xp[..., R:R + N], xp[..., R + N:]")],
    "dt_bias_outside_softplus": [("delta_bias=W[\"dt_bias\"], D=W[\"D\"]", "D=W[\"D\"]")],
    "conv_taps_reversed": [("c += conv_w[:, k] * full[:, k:k + L, :]", "c += conv_w[:, K - 1 - k] * full[:, k:k + L, :]")],
    "projections_read_pre_conv": [("xp = u @ np.asarray(W[\"W_x\"], np.float64).T", "xp = xi @ np.asarray(W[\"W_x\"], np.float64).T")],
    "history_not_returned": [("return silu(c), np.ascontiguousarray(np.transpose(full[:, L:, :], (0, 2, 1)))",
                              "return silu(c), np.ascontiguousarray(np.transpose(full[:, :K - 1, :], (0, 2, 1)))")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_mutant_is_caught(name, tmp_path):
    src = open(oracle.block.__file__).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
        src = src.replace(old, new)
    # the mutant lives in a copy of the package so that its relative import works
    pkg = tmp_path / "oracle_mut"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(
        "from oracle import default, Oracle  # noqa: F401\n")
    (pkg / "block.py").write_text(src)
    sys.path.insert(0, str(tmp_path))
    try:
        spec = importlib.util.spec_from_file_location("oracle_mut.block", pkg / "block.py",
                                                      submodule_search_locations=None)
        importlib.import_module("oracle_mut")
        mod = importlib.util.module_from_spec(spec)
        mod.__package__ = "oracle_mut"
        spec.loader.exec_module(mod)
    finally:
        sys.path.remove(str(tmp_path))
        sys.modules.pop("oracle_mut", None)
    caught = []
    for pin in pins_block.BLOCK_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
