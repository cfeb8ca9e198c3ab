"""The sequence-parallel oracle against its pins, and planted mistakes that a pin must catch (CPU only)."""
import inspect
import types

import pytest

from oracle import sp
from tests import pins_sp

MUTATIONS = {
    "philox_key_bump_first_round": ("        if r > 0:\n            k0 =", "        if r >= 0:\n            k0 ="),
    "philox_swapped_multipliers": ("p0 = m0 * c[:, 0]", "p0 = m1 * c[:, 0]"),
    "philox_dropped_xor": ("hi1 ^ c[:, 1] ^ k0", "hi1 ^ k0"),
    "mask_ignores_row0": ("n0 = row0 * h // 4", "n0 = 0"),
    "mask_inverted": ("return words >= np.uint32(keep_threshold(p))", "return words < np.uint32(keep_threshold(p))"),
    "dropout_unscaled": ("return 1.0 / (1.0 - float(np.float32(p)))", "return 1.0"),
    "ln_unbiased_variance": ("var = ((X - mu[:, None]) ** 2).sum(axis=1) / h",
                             "var = ((X - mu[:, None]) ** 2).sum(axis=1) / (h - 1)"),
    "ln_eps_outside_sqrt": ("rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / (np.sqrt(var) + eps)"),
    "ln_beta_dropped": ("* xhat + np.asarray(beta, dtype=np.float64)[None, :]", "* xhat"),
    "ln_bwd_dropped_mean_term": ("(g - g.mean(axis=1, keepdims=True) - xh *", "(g - xh *"),
    "ln_dgamma_wrong": ("\"dgamma\": (dY * xh).sum(axis=0)", "\"dgamma\": dY.sum(axis=0)"),
    "residual_dropped": ("return np.asarray(residual, dtype=np.float64) + np.where(keep, z * dropout_scale(p), 0.0)",
                         "return np.where(keep, z * dropout_scale(p), 0.0)"),
    # The same mistake made in both oracle paths (the reduce-scatter end and
    # the whole-sequence block), which pin each other: only the torch forward
    # pin can catch these.
    "dropout_after_residual_both": [
        ("return np.asarray(residual, dtype=np.float64) + np.where(keep, z * dropout_scale(p), 0.0)",
         "return np.where(keep, (np.asarray(residual, dtype=np.float64) + z) * dropout_scale(p), 0.0)"),
        ('"out": np.asarray(X, dtype=np.float64) + np.where(keep, Z * dropout_scale(p), 0.0)',
         '"out": np.where(keep, (np.asarray(X, dtype=np.float64) + Z) * dropout_scale(p), 0.0)')],
    "residual_scaled_both": [
        ("return np.asarray(residual, dtype=np.float64) + np.where(keep, z * dropout_scale(p), 0.0)",
         "return np.asarray(residual, dtype=np.float64) * dropout_scale(p) + np.where(keep, z * dropout_scale(p), 0.0)"),
        ('"out": np.asarray(X, dtype=np.float64) + np.where(keep, Z * dropout_scale(p), 0.0)',
         '"out": np.asarray(X, dtype=np.float64) * dropout_scale(p) + np.where(keep, Z * dropout_scale(p), 0.0)')],
}


@pytest.mark.parametrize("pin", pins_sp.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(sp)


def _mutant(name, edits):
    """The oracle with each (old, new) edit applied once; edits may be one pair or a list of pairs."""
    src = inspect.getsource(sp)
    for old, new in ([edits] if isinstance(edits, tuple) else edits):
        assert src.count(old) >= 1, f"mutation {name} does not apply"
        src = src.replace(old, new, 1)
    mod = types.ModuleType(f"sp_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_pin_catches(name):
    mod = _mutant(name, MUTATIONS[name])
    caught = []
    for pin in pins_sp.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"


@pytest.mark.parametrize("name", ["dropout_after_residual_both", "residual_scaled_both"])
def test_consistent_mistakes_need_the_torch_forward_pin(name):
    """Without pin_sp_forward_torch these two-place mistakes pass every other pin."""
    mod = _mutant(name, MUTATIONS[name])
    others = [p for p in pins_sp.ALL_PINS if p is not pins_sp.pin_sp_forward_torch]
    for pin in others:
        pin(mod)
    with pytest.raises(AssertionError):
        pins_sp.pin_sp_forward_torch(mod)
