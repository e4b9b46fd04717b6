"""Plants one plausible mistake at a time in a copy of the oracle (on the CPU)
and checks that the pins catch it: a dropped term, a wrong sign, base or
index, a transposed operand, a mask that lets padding in.  Each mutated copy
must fail at least one pin; the unmutated copy must pass them all."""
import importlib.util
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "sigattn_oracle.py")

MUTATIONS = {
    "bias_sign": ("return -math.log(n)", "return math.log(n)"),
    "bias_log10": ("return -math.log(n)", "return -math.log10(n)"),
    "bias_uses_lmax": ("b = bias(n, bias_mode, bias_arg) if", "b = bias(L, bias_mode, bias_arg) if"),
    "dbias_sums_over_keys": ('it["dx"].sum(axis=0)', 'it["dx"].sum(axis=1)'),
    "dbias_uses_dp": ('it["dx"].sum(axis=0)', 'it["dp"].sum(axis=0)'),
    "dbias_uses_p": ('it["dx"].sum(axis=0)', 'it["p"].sum(axis=0)'),
    "per_head_bias_first_head": ("return float(vals[h])", "return float(vals[0])"),
    "per_head_bias_negated": ("return float(vals[h])", "return -float(vals[h])"),
    "scale_1_over_d": ("return 1.0 / math.sqrt(d)", "return 1.0 / d"),
    "scale_dropped": ("x = s * (q @ k.T) + b          # scores", "x = (q @ k.T) + b          # scores"),
    "scores_transposed": ("x = s * (q @ k.T) + b          # scores", "x = s * (k @ q.T) + b          # scores"),
    "pv_transposed": ("return p @ v", "return p.T @ v"),
    "logistic_neg_branch": ("out[~pos] = e / (1.0 + e)", "out[~pos] = 1.0 / (1.0 + e)"),
    "logistic_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(x[pos]))"),
    "dv_not_transposed": ("dv = p.T @ do", "dv = p @ do"),
    "dp_transposed": ("dp = do @ v.T", "dp = (do @ v.T).T"),
    "dsigma_dropped": ("dx = dp * (p * logistic(-x))", "dx = dp * p"),
    "dsigma_sign": ("dx = dp * (p * logistic(-x))", "dx = dp * (p * logistic(x))"),
    "dq_transposed": ("dq = s * (dx @ k)", "dq = s * (dx.T @ k)"),
    "dq_scale_dropped": ("dq = s * (dx @ k)", "dq = (dx @ k)"),
    "dk_not_transposed": ("dk = s * (dx.T @ q)", "dk = s * (dx @ q)"),
    "dk_uses_k": ("dk = s * (dx.T @ q)", "dk = s * (dx.T @ k)"),
    "keys_include_padding": ("qv, kv, vv = q[bi, h, :n], k[bi, h, :n], v[bi, h, :n]",
                             "qv, kv, vv = q[bi, h, :n], k[bi, h, :n + 1], v[bi, h, :n + 1]"),
    "causal_mask_transposed": ("return np.tril(np.ones((n, n)))", "return np.triu(np.ones((n, n)))"),
    "causal_forward_only": ("    if causal:  # masked weights are constants 0: no gradient through them\n        p = p * causal_mask(q.shape[0])\n", ""),
    "head_drops_last_row": ("o[:n] = head_forward(q[:n], k[:n], v[:n], b)",
                            "o[:n - 1] = head_forward(q[:n], k[:n], v[:n], b)[:n - 1]"),
}


def _load(src: str) -> types.ModuleType:
    spec = importlib.util.spec_from_loader("mutated_oracle", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "mutated_oracle", "exec"), mod.__dict__)
    return mod


def _failures(mod):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # an assertion, a shape error or a raised warning all count
            failed.append(pin.__name__)
    return failed


with open(SRC_PATH) as f:
    SOURCE = f.read()


def test_unmutated_copy_passes():
    assert _failures(_load(SOURCE)) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    assert SOURCE.count(old) >= 1, f"mutation anchor for {name} not found in the oracle"
    mod = _load(SOURCE.replace(old, new, 1))
    assert _failures(mod), f"no pin caught mutation {name}"
