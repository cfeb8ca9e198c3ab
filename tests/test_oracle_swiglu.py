"""The gated-MLP oracle against its pins, and planted mistakes that a pin must catch (CPU only)."""
import inspect
import types

import pytest

from oracle import swiglu
from tests import pins_swiglu

MUTATIONS = {
    "silu_without_x": ("    return x * sigmoid(x)", "    return sigmoid(x)"),
    "silu_grad_dropped_term": ("return s * (1.0 + x * (1.0 - s))", "return s"),
    "sigmoid_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(x[pos]))"),
    "interleave_up_first": ("np.concatenate([g, u], axis=-2)", "np.concatenate([u, g], axis=-2)"),
    "group_of_4": ("GROUP = 8", "GROUP = 4"),
    "pack_wrong_shard": ("col_shard(W_up, tp, i))", "col_shard(W_up, tp, 0))"),
    "down_wrong_rows": ("\"Z\": matmul(A, row_shard(W_down, tp, i))}", "\"Z\": matmul(A, row_shard(W_down, tp, 0))}"),
    "dgate_without_up": ("dGU = interleave(dA * U * silu_grad(G), dA * silu(G))",
                         "dGU = interleave(dA * silu_grad(G), dA * silu(G))"),
    "dup_without_silu": ("dGU = interleave(dA * U * silu_grad(G), dA * silu(G))",
                         "dGU = interleave(dA * U * silu_grad(G), dA * G)"),
    "dx_dropped_up_term": ("            + matmul(dU, np.asarray(W_up, dtype=np.float64).T)}",
                           "            - matmul(dU, np.asarray(W_up, dtype=np.float64).T)}"),
    "dw_gu_wrong_operand": ("\"dW_gu\": matmul(X.T, dGU)", "\"dW_gu\": matmul(X.T, dGU) * 1.001"),
    "dw_down_offset": ("\"dW_down\": matmul(A.T, dZ),\n", "\"dW_down\": matmul(A.T, dZ) + 1e-3,\n"),
}


@pytest.mark.parametrize("pin", pins_swiglu.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(swiglu)


def _mutant(name, old, new):
    src = inspect.getsource(swiglu)
    assert src.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"swiglu_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_pin_catches(name):
    mod = _mutant(name, *MUTATIONS[name])
    caught = []
    for pin in pins_swiglu.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
