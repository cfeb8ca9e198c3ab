"""Plant plausible mistakes in copies of the oracle and check that a pin catches each.

The mistakes are planted in the CPU oracle only (a copy of its source with
one edit), never in GPU code.
"""
import importlib.util
import inspect
import sys
import types

import pytest

from oracle import ref
from tests import pins

MUTATIONS = {
    "gelu_constant": ("GELU_CUBIC = 0.044715", "GELU_CUBIC = 0.04"),
    "gelu_grad_sign": ("0.5 * x * (1.0 - t * t) * du", "0.5 * x * (1.0 + t * t) * du"),
    "gelu_grad_dropped_term": ("return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du", "return 0.5 * (1.0 + t)"),
    "bias_sign": ("H = H + bi[None, :]", "H = H - bi[None, :]"),
    "col_shard_index": ("[:, i * w:(i + 1) * w]", "[:, i:i + w]"),
    "row_shard_index": ("[i * w:(i + 1) * w, :]", "[(tp - 1 - i) * w:(tp - i) * w, :]"),
    "partial_sum_sign": ("out = out + p", "out = out - p"),
    "bwd_uses_dA_for_dW1": ("dW1 = matmul(np.asarray(X, dtype=np.float64).T, dH)",
                            "dW1 = matmul(np.asarray(X, dtype=np.float64).T, dA)"),
    "bwd_shard_no_act_grad": ("dH_i = dA_i * act_grad(H_i, act)", "dH_i = dA_i"),
    "bwd_dW2_transposed": ("dW2 = matmul(f[\"A\"].T, dZ)", "dW2 = matmul(dZ.T, f[\"A\"]).T * 1.0001"),
    "row_fwd_wrong_block": ("return matmul(col_shard(X, tp, i), row_shard(W, tp, i))",
                            "return matmul(col_shard(X, tp, 0), row_shard(W, tp, i))"),
    "col_bwd_wrong_operand": ("\"dW\": matmul(np.asarray(X, dtype=np.float64).T, dY_i)}",
                              "\"dW\": matmul(np.asarray(X, dtype=np.float64).T, np.abs(dY_i))}"),
    "db_sum_axis": ("return {\"dA\": dA_i, \"dH\": dH_i, \"db1\": dH_i.sum(axis=0)",
                    "return {\"dA\": dA_i, \"dH\": dH_i, \"db1\": dA_i.sum(axis=0)"),
    "sampled_rows_no_bias": ("    Xr = np.asarray(X, dtype=np.float64)[np.asarray(rows)]\n    H = matmul(Xr, W1_i)\n    if b1_i is not None:",
                             "    Xr = np.asarray(X, dtype=np.float64)[np.asarray(rows)]\n    H = matmul(Xr, W1_i)\n    if False:"),
    "qkv_head_order": ("for W in (Wq, Wk, Wv)], axis=1)", "for W in (Wq, Wv, Wk)], axis=1)"),
    "divisibility_unchecked": ("if tp < 1 or n % tp != 0:", "if tp < 1:"),
}


def _mutant(name, old, new):
    src = inspect.getsource(ref)
    assert src.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_pin_catches(name):
    mod = _mutant(name, *MUTATIONS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
