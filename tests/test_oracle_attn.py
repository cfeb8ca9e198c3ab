"""The attention oracle against its pins, and planted mistakes that a pin must catch (CPU only)."""
import inspect
import types

import pytest

from oracle import attn
from tests import pins_attn

MUTATIONS = {
    "causal_off_by_one": ("np.triu(np.ones((seq, seq), dtype=bool), k=1)", "np.triu(np.ones((seq, seq), dtype=bool), k=2)"),
    "no_scale": ("S = np.matmul(q, k.transpose(0, 1, 3, 2)) * scale", "S = np.matmul(q, k.transpose(0, 1, 3, 2))"),
    "softmax_wrong_axis": ("l = E.sum(axis=-1, keepdims=True)\n    P = E / l", "l = E.sum(axis=-2, keepdims=True)\n    P = E / l"),
    "lse_without_log": ("lse = (m + np.log(l))[..., 0]", "lse = (m + l)[..., 0]"),
    "D_from_values": ("D = (do * o).sum(axis=-1, keepdims=True)", "D = (do * v).sum(axis=-1, keepdims=True)"),
    "dK_unscaled": ("dK = np.matmul(dS.transpose(0, 1, 3, 2), q) * scale", "dK = np.matmul(dS.transpose(0, 1, 3, 2), q)"),
    "dV_untransposed": ("dV = np.matmul(P.transpose(0, 1, 3, 2), do)", "dV = np.matmul(P, do)"),
    "dS_missing_D": ("\n    dS = P * (dP - D)\n", "\n    dS = P * dP\n"),
    "heads_interleaved": ("return M.reshape(batch, seq, heads, d).transpose(0, 2, 1, 3)",
                          "return M.reshape(batch, seq, d, heads).transpose(0, 3, 1, 2)"),
    "block_shard_by_heads_not_columns": ("return slice(i * w, (i + 1) * w)",
                                         "return slice(i * (heads // tp), i * (heads // tp) + w)"),
    "block_dO_from_Wo_columns": ("dO = dZ @ Wo_i.T", "dO = dZ @ np.asarray(Wo, dtype=np.float64)[:, c].T"),
    "block_dX_from_queries_only": ('"dX": dQKV @ Wqkv.T', '"dX": dQKV[:, :w] @ Wqkv[:, :w].T'),
}


@pytest.mark.parametrize("pin", pins_attn.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(attn)


def _mutant(name, old, new):
    src = inspect.getsource(attn)
    assert src.count(old) >= 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"attn_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_pin_catches(name):
    mod = _mutant(name, *MUTATIONS[name])
    caught = []
    for pin in pins_attn.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
