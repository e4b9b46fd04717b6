"""The softmax oracle against its pins, and planted mistakes (in copies of
the oracle, on the CPU) that the pins must catch."""
import importlib.util
import os
import types

import pytest

from oracle import softmax_oracle
from softmax_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "softmax_oracle.py")
with open(SRC_PATH) as f:
    SOURCE = f.read()

MUTATIONS = {
    "no_row_max_in_lse": ("return (m + np.log(", "return (np.log("),
    "normalise_columns": ("return e / np.sum(e, axis=-1, keepdims=True)", "return e / np.sum(e, axis=0, keepdims=True)"),
    "scale_dropped": ("x = _masked((q @ k.T) / math.sqrt(q.shape[1]), causal)", "x = _masked((q @ k.T), causal)"),
    "pv_transposed": ("return p @ v, row_logsumexp(x)", "return p.T @ v, row_logsumexp(x)"),
    "jacobian_row_term_dropped": ("dx = p * (dp - row)", "dx = p * dp"),
    "jacobian_wrong_axis": ("row = np.sum(p * dp, axis=-1, keepdims=True)",
                            "row = np.sum(p * dp, axis=0, keepdims=True)"),
    "row_term_from_dp_only": ("row = np.sum(p * dp, axis=-1, keepdims=True)",
                              "row = np.sum(dp, axis=-1, keepdims=True)"),
    "dv_not_transposed": ("dv = p.T @ do", "dv = p @ do"),
    "dk_uses_k": ("return s * (dx @ k), s * (dx.T @ q), dv", "return s * (dx @ k), s * (dx.T @ k), dv"),
    "causal_mask_transposed": ("np.where(np.tril(np.ones((n, n))) > 0, x, -np.inf)", "np.where(np.triu(np.ones((n, n))) > 0, x, -np.inf)"),
    "causal_backward_unmasked": ("x = _masked(s * (q @ k.T), causal)", "x = s * (q @ k.T)"),
    "keys_include_padding": ("qv, kv, vv = q[bi, h, :n], k[bi, h, :n], v[bi, h, :n]",
                             "qv, kv, vv = q[bi, h, :n], k[bi, h, :n + 1], v[bi, h, :n + 1]"),
}


def _load(src):
    spec = importlib.util.spec_from_loader("mutated_softmax_oracle", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "mutated_softmax_oracle", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(softmax_oracle)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) == 1, name
    mod = _load(SOURCE.replace(old, new))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
