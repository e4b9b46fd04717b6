"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes the oracle module as its argument and raises AssertionError on
a mismatch, so the same pins run against the real oracle (test_oracle_pins.py)
and against copies of it with a planted mistake (test_oracle_mutations.py),
which must each fail at least one pin.

What the pins rest on (pages: "Better Models, Faster Training: Sigmoid
Attention for single-cell Foundation Models", summary §2A/§2B, and its
abstract on the paperdance card):
  * closed forms of the §2A formula: a zero query (or key) makes every score
    equal to the bias, so every valid weight is sigma(-ln n) = 1/(n+1);
  * a single key (n = 1, bias 0) reduces to the textbook logistic of q.k/sqrt(d);
  * a one-hot V reads out one column of the weight matrix, which fixes the
    orientation of P and the 1/sqrt(d) scale against scipy's logistic;
  * brute-force scalar loops on tiny inputs;
  * the backward: central finite differences of l = sum(O * dO), and torch
    autograd of an independently written forward;
  * sigma' <= 1/4 with equality at 0 (§2B), dO = 0 => zero gradients;
  * padding carries no information (§2C block skip), n = 0 gives zeros;
  * permuting the valid keys (K and V together) leaves O unchanged.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"


def pin_zero_query_uniform_weights(O):
    """Q = 0 => O_i = sum_{j<n} V_j / (n + 1) on valid rows, 0 on padded rows."""
    B, H, L, d = 3, 2, 12, 8
    seqlens = [12, 5, 1]
    for zero in ("q", "k"):
        q, k, v = _rand((B, H, L, d), 1), _rand((B, H, L, d), 2), _rand((B, H, L, d), 3)
        if zero == "q":
            q[:] = 0.0
        else:
            k[:] = 0.0
        o = O.attention(q, k, v, seqlens)["o"]
        for b, n in enumerate(seqlens):
            want = v[b, :, :n].sum(axis=1, keepdims=True) / (n + 1)
            _close(o[b, :, :n], np.broadcast_to(want, (H, n, d)), what=f"{zero}=0 b={b}")
            assert np.all(o[b, :, n:] == 0.0), "padded rows must be 0"


def pin_unit_values_row_sums(O):
    """V = 1 => every column of O_i equals the row sum of weights; with Q = 0
    that row sum is n/(n+1)."""
    B, H, L, d = 2, 2, 9, 4
    seqlens = [9, 4]
    q, k = _rand((B, H, L, d), 4), _rand((B, H, L, d), 5)
    v = np.ones((B, H, L, d))
    o = O.attention(q, k, v, seqlens)["o"]
    for b, n in enumerate(seqlens):
        cols = o[b, :, :n]
        _close(cols, np.broadcast_to(cols[..., :1], cols.shape), what="columns equal")
        assert np.all(cols > 0) and np.all(cols < n), "row sums of weights lie in (0, n)"
    o0 = O.attention(np.zeros_like(q), k, v, seqlens)["o"]
    for b, n in enumerate(seqlens):
        _close(o0[b, :, :n], np.full((H, n, d), n / (n + 1)), what="n/(n+1)")


def pin_single_key_textbook_logistic(O):
    """n = 1 => b = -ln 1 = 0 and O_0 = sigma(q.k/sqrt(d)) v (scipy's expit)."""
    d = 16
    for seed in range(5):
        q, k, v = _rand((1, 1, 3, d), 10 + seed, 2.0), _rand((1, 1, 3, d), 20 + seed), _rand((1, 1, 3, d), 30 + seed)
        o = O.attention(q, k, v, [1])["o"]
        w = scipy.special.expit(float(np.dot(q[0, 0, 0], k[0, 0, 0])) / math.sqrt(d))
        _close(o[0, 0, 0], w * v[0, 0, 0], what="single key")
        assert np.all(o[0, 0, 1:] == 0.0)


def pin_one_hot_value_reads_weight_column(O):
    """V_j = e_c for j = j*, else 0 => O[i, c] = sigma(q_i.k_j*/sqrt(d) - ln n)."""
    L, d, n, c = 10, 8, 7, 3
    q, k = _rand((1, 1, L, d), 40, 1.5), _rand((1, 1, L, d), 41, 1.5)
    for jstar in (0, 4, 6):
        v = np.zeros((1, 1, L, d))
        v[0, 0, jstar, c] = 1.0
        o = O.attention(q, k, v, [n])["o"][0, 0]
        for i in range(n):
            x = sum(q[0, 0, i, t] * k[0, 0, jstar, t] for t in range(d)) / math.sqrt(d) - math.log(n)
            assert abs(o[i, c] - scipy.special.expit(x)) <= 1e-13, (i, jstar)
            others = np.delete(o[i], c)
            assert np.all(others == 0.0)


def _brute_forward(q, k, v, n, b):
    """Scalar loops on the valid block, textbook logistic."""
    d = len(q[0])
    out = [[0.0] * d for _ in range(n)]
    for i in range(n):
        for j in range(n):
            x = sum(q[i][t] * k[j][t] for t in range(d)) / math.sqrt(d) + b
            w = 1.0 / (1.0 + math.exp(-x))
            for c in range(d):
                out[i][c] += w * v[j][c]
    return out


def pin_brute_force_tiny(O):
    """Vectorised oracle == scalar loops, several tiny ragged batches."""
    for seed, (B, H, L, d, seqlens) in enumerate([(2, 2, 6, 4, [6, 3]), (3, 1, 5, 3, [1, 5, 2])]):
        q, k, v = _rand((B, H, L, d), 50 + seed), _rand((B, H, L, d), 60 + seed), _rand((B, H, L, d), 70 + seed)
        o = O.attention(q, k, v, seqlens)["o"]
        for b, n in enumerate(seqlens):
            for h in range(H):
                want = _brute_forward(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), n, -math.log(n))
                _close(o[b, h, :n], np.array(want), what=f"brute b={b} h={h}")
                assert np.all(o[b, h, n:] == 0.0)


def pin_backward_finite_differences(O):
    """Central differences of l = sum over valid rows of O * dO (h = 1e-6)."""
    B, H, L, d = 2, 1, 7, 4
    seqlens = [5, 7]
    q, k, v = _rand((B, H, L, d), 80), _rand((B, H, L, d), 81), _rand((B, H, L, d), 82)
    do = _rand((B, H, L, d), 83)

    def loss(q_, k_, v_):
        o = O.attention(q_, k_, v_, seqlens)["o"]
        return float((o * do).sum())  # padded rows of O are 0, so dO there is ignored

    g = O.attention(q, k, v, seqlens, do=do)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            key = name[1]
            xp = args[key].copy()
            xm = args[key].copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args), dict(args)
            ap[key], am[key] = xp, xm
            num[idx] = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(g[name] - num).max() <= 1e-7 * scale, f"{name}: FD mismatch {np.abs(g[name] - num).max():.3e}"
        for b, n in enumerate(seqlens):
            assert np.all(g[name][b, :, n:] == 0.0), f"{name} padded rows must be 0"


def pin_backward_autograd(O):
    """torch fp64 autograd of sigmoid(Q K^T / sqrt(d) - ln n) V on each valid block."""
    B, H, L, d = 2, 3, 16, 8
    seqlens = [16, 11]
    q, k, v, do = (_rand((B, H, L, d), 90 + i) for i in range(4))
    got = O.attention(q, k, v, seqlens, do=do)
    for b, n in enumerate(seqlens):
        for h in range(H):
            tq = torch.tensor(q[b, h, :n], requires_grad=True)
            tk = torch.tensor(k[b, h, :n], requires_grad=True)
            tv = torch.tensor(v[b, h, :n], requires_grad=True)
            w = torch.sigmoid(tq @ tk.transpose(0, 1) / math.sqrt(d) - math.log(n))
            out = w @ tv
            (out * torch.tensor(do[b, h, :n])).sum().backward()
            _close(got["o"][b, h, :n], out.detach().numpy(), rtol=1e-12, atol=1e-12, what="autograd O")
            _close(got["dq"][b, h, :n], tq.grad.numpy(), rtol=1e-11, atol=1e-12, what="autograd dQ")
            _close(got["dk"][b, h, :n], tk.grad.numpy(), rtol=1e-11, atol=1e-12, what="autograd dK")
            _close(got["dv"][b, h, :n], tv.grad.numpy(), rtol=1e-11, atol=1e-12, what="autograd dV")


def pin_derivative_bound(O):
    """|dX| <= |dP| / 4 everywhere (summary §2B), with equality where X = 0."""
    n, d = 9, 8
    q, k, v, do = (_rand((n, d), 100 + i, 3.0) for i in range(4))
    _, _, _, it = O.head_backward(q, k, v, do, O.bias(n), intermediates=True)
    assert np.all(np.abs(it["dx"]) <= 0.25 * np.abs(it["dp"]) * (1 + 1e-15))
    # X = 0 everywhere: zero queries and a zero constant bias.
    _, _, _, it0 = O.head_backward(np.zeros((n, d)), k, v, do, O.bias(n, "const", 0.0), intermediates=True)
    _close(it0["dx"], 0.25 * it0["dp"], rtol=1e-15, atol=0.0, what="equality at 0")


def pin_zero_dout_zero_grads(O):
    B, H, L, d = 2, 2, 8, 4
    q, k, v = (_rand((B, H, L, d), 110 + i) for i in range(3))
    g = O.attention(q, k, v, [8, 3], do=np.zeros((B, H, L, d)))
    for key in ("dq", "dk", "dv"):
        assert np.all(g[key] == 0.0)


def pin_padding_carries_nothing(O):
    """Overwriting padded rows of Q/K/V/dO (other values, +-inf, nan) leaves
    valid outputs bitwise unchanged; padded output rows stay exactly 0."""
    B, H, L, d = 3, 2, 10, 4
    seqlens = [10, 6, 0]
    q, k, v, do = (_rand((B, H, L, d), 120 + i) for i in range(4))
    ref = O.attention(q, k, v, seqlens, do=do)
    for fill in ("other", "inf", "nan"):
        q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
        for b, n in enumerate(seqlens):
            for t, x in enumerate((q2, k2, v2, do2)):
                if fill == "other":
                    x[b, :, n:] = _rand(x[b, :, n:].shape, 130 + t + b, 7.0)
                elif fill == "inf":
                    x[b, :, n:] = np.inf if t % 2 else -np.inf
                else:
                    x[b, :, n:] = np.nan
        with np.errstate(all="raise"):
            got = O.attention(q2, k2, v2, seqlens, do=do2)
        for key in ("o", "dq", "dk", "dv"):
            assert np.array_equal(got[key], ref[key]), f"{key} changed with padded {fill}"
            for b, n in enumerate(seqlens):
                assert np.all(got[key][b, :, n:] == 0.0)


def pin_key_permutation(O):
    """Permuting valid keys (K and V rows together) leaves O and dQ unchanged
    and permutes dK, dV the same way."""
    L, d, n = 12, 8, 10
    q, k, v, do = (_rand((1, 1, L, d), 140 + i) for i in range(4))
    perm = np.random.default_rng(7).permutation(n)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, :n] = k[0, 0, perm]
    v2[0, 0, :n] = v[0, 0, perm]
    a = O.attention(q, k, v, [n], do=do)
    b = O.attention(q, k2, v2, [n], do=do)
    _close(b["o"], a["o"], what="O perm")
    _close(b["dq"], a["dq"], what="dQ perm")
    _close(b["dk"][0, 0, :n], a["dk"][0, 0, perm], what="dK perm")
    _close(b["dv"][0, 0, :n], a["dv"][0, 0, perm], what="dV perm")


def pin_zero_length_sequence(O):
    B, H, L, d = 2, 2, 6, 4
    q, k, v, do = (_rand((B, H, L, d), 150 + i) for i in range(4))
    with np.errstate(all="raise"):
        g = O.attention(q, k, v, [0, 0], do=do)
        o, dq, dk, dv = O.head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0)
    for key in g:
        assert np.all(g[key] == 0.0)
    for x in (o, dq, dk, dv):
        assert np.all(x == 0.0)


def pin_logistic(O):
    """sigma(x) = (1 + tanh(x/2))/2, sigma(0) = 1/2, no overflow at +-1000,
    and agreement with scipy's expit."""
    x = np.linspace(-700, 700, 200001)
    s = O.logistic(x)
    assert np.abs(s - 0.5 * (1.0 + np.tanh(0.5 * x))).max() <= 1e-15
    assert O.logistic(np.array([0.0]))[0] == 0.5
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        big = O.logistic(np.array([-1000.0, 1000.0]))
    assert big[0] == 0.0 and big[1] == 1.0
    ref = scipy.special.expit(x)
    assert np.all(np.abs(s - ref) <= 1e-15 * np.maximum(ref, 1e-300) + 1e-300)


def pin_bias_modes(O):
    """fixed_n: weights 1/(N+1) under Q = 0; const: weights sigma(b)."""
    B, H, L, d = 2, 1, 8, 4
    seqlens = [8, 3]
    k, v = _rand((B, H, L, d), 160), _rand((B, H, L, d), 161)
    q = np.zeros((B, H, L, d))
    o = O.attention(q, k, v, seqlens, bias_mode="fixed_n", bias_arg=100.0)["o"]
    for b, n in enumerate(seqlens):
        _close(o[b, :, :n], np.broadcast_to(v[b, :, :n].sum(1, keepdims=True) / 101.0, (H, n, d)), what="fixed_n")
    o = O.attention(q, k, v, seqlens, bias_mode="const", bias_arg=0.75)["o"]
    w = scipy.special.expit(0.75)
    for b, n in enumerate(seqlens):
        _close(o[b, :, :n], np.broadcast_to(w * v[b, :, :n].sum(1, keepdims=True), (H, n, d)), what="const")


def pin_linear_in_values(O):
    """O is linear in V: O(V1 + 2 V2) = O(V1) + 2 O(V2)."""
    B, H, L, d = 1, 2, 9, 4
    q, k, v1, v2 = (_rand((B, H, L, d), 170 + i) for i in range(4))
    f = lambda v: O.attention(q, k, v, [7])["o"]
    _close(f(v1 + 2 * v2), f(v1) + 2 * f(v2), rtol=1e-12, atol=1e-12, what="linearity")


def pin_head_matches_batch(O):
    """The per-head sampling route returns the same rows as the batch route."""
    B, H, L, d = 2, 2, 10, 4
    seqlens = [10, 6]
    q, k, v, do = (_rand((B, H, L, d), 180 + i) for i in range(4))
    g = O.attention(q, k, v, seqlens, do=do)
    for b, n in enumerate(seqlens):
        for h in range(H):
            o, dq, dk, dv = O.head(q[b, h], k[b, h], v[b, h], do[b, h], n)
            for key, x in zip(("o", "dq", "dk", "dv"), (o, dq, dk, dv)):
                assert np.array_equal(x, g[key][b, h]), key


ALL_PINS = [
    pin_zero_query_uniform_weights,
    pin_unit_values_row_sums,
    pin_single_key_textbook_logistic,
    pin_one_hot_value_reads_weight_column,
    pin_brute_force_tiny,
    pin_backward_finite_differences,
    pin_backward_autograd,
    pin_derivative_bound,
    pin_zero_dout_zero_grads,
    pin_padding_carries_nothing,
    pin_key_permutation,
    pin_zero_length_sequence,
    pin_logistic,
    pin_bias_modes,
    pin_linear_in_values,
    pin_head_matches_batch,
]


# --- causal variant -----------------------------------------------------------

def pin_causal_zero_query(O):
    """Causal, Q = 0: every visible weight is 1/(n+1), so O_i = sum_{j<=i} V_j / (n+1)."""
    B, H, L, d = 2, 2, 10, 4
    seqlens = [10, 6]
    v = _rand((B, H, L, d), 41)
    q, k = np.zeros_like(v), _rand((B, H, L, d), 42)
    o = O.attention(q, k, v, seqlens, causal=True)["o"]
    for b, n in enumerate(seqlens):
        want = np.cumsum(v[b, :, :n], axis=1) / (n + 1)
        _close(o[b, :, :n], want, what=f"causal q=0 b={b}")
        assert np.all(o[b, :, n:] == 0.0)


def pin_causal_brute_force(O):
    """Scalar loops over j <= i with math.exp, forward and (via the loss) dV."""
    L, d = 6, 3
    q, k, v, do = (_rand((1, 1, L, d), s) for s in (43, 44, 45, 46))
    n = 5
    out = O.attention(q, k, v, [n], do=do, causal=True)
    b = -math.log(n)
    for i in range(n):
        for c in range(d):
            acc = 0.0
            for j in range(i + 1):
                x = sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) / math.sqrt(d) + b
                acc += v[0, 0, j, c] / (1.0 + math.exp(-x))
            assert abs(out["o"][0, 0, i, c] - acc) < 1e-12
    for j in range(n):  # dV_j = sum_{i >= j} P_ij dO_i
        for c in range(d):
            acc = 0.0
            for i in range(j, n):
                x = sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) / math.sqrt(d) + b
                acc += do[0, 0, i, c] / (1.0 + math.exp(-x))
            assert abs(out["dv"][0, 0, j, c] - acc) < 1e-12


def pin_causal_prefix(O):
    """Rows after i of K and V cannot change O_i (nor dQ_i)."""
    L, d = 9, 4
    q, k, v, do = (_rand((1, 2, L, d), s) for s in (47, 48, 49, 50))
    a = O.attention(q, k, v, [9], do=do, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:] += 3.0
    v2[:, :, 5:] -= 2.0
    b = O.attention(q, k2, v2, [9], do=do, causal=True)
    _close(a["o"][:, :, :5], b["o"][:, :, :5], what="causal prefix O")
    _close(a["dq"][:, :, :5], b["dq"][:, :, :5], what="causal prefix dQ")


def pin_causal_finite_differences(O):
    """Central differences of l = sum(O * dO) in the causal variant."""
    L, d = 4, 2
    q, k, v, do = (_rand((1, 1, L, d), s) for s in (51, 52, 53, 54))
    g = O.attention(q, k, v, [L], do=do, causal=True)
    h = 1e-6
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        base = {"q": q, "k": k, "v": v}
        for idx in np.ndindex(base[name].shape):
            xp, xm = dict(base), dict(base)
            xp[name] = base[name].copy()
            xm[name] = base[name].copy()
            xp[name][idx] += h
            xm[name][idx] -= h
            lp = np.sum(O.attention(xp["q"], xp["k"], xp["v"], [L], causal=True)["o"] * do)
            lm = np.sum(O.attention(xm["q"], xm["k"], xm["v"], [L], causal=True)["o"] * do)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[key][idx]) < 1e-7 * (1 + abs(fd)), (name, idx)


ALL_PINS += [pin_causal_zero_query, pin_causal_brute_force, pin_causal_prefix, pin_causal_finite_differences]


# --- learnable per-head bias and its gradient -------------------------------

def pin_dbias_zero_scores_closed_form(O):
    """Q = K = 0 makes every score equal to the head's bias b_h, so
    dX_ij = sigma'(b_h) (dO_i . V_j) and the per-key sum over queries is
    sigma'(b_h) (sum_i dO_i) . V_j (over i >= j in the causal variant);
    sigma' from scipy's logistic."""
    B, H, L, d = 2, 2, 7, 3
    seqlens = [7, 4]
    vals = np.array([0.4, -1.3])
    v, do = _rand((B, H, L, d), 61), _rand((B, H, L, d), 62)
    q = k = np.zeros((B, H, L, d))
    for causal in (False, True):
        g = O.attention(q, k, v, seqlens, do=do, bias_mode="per_head", bias_arg=vals, causal=causal)
        for b, n in enumerate(seqlens):
            for h in range(H):
                sp = scipy.special.expit(vals[h]) * scipy.special.expit(-vals[h])
                for j in range(n):
                    rows = range(j, n) if causal else range(n)
                    want = sp * sum(float(do[b, h, i] @ v[b, h, j]) for i in rows)
                    assert abs(g["dbias"][b, h, j] - want) < 1e-12, (causal, b, h, j)
            assert np.all(g["dbias"][b, :, n:] == 0.0)


def pin_dbias_finite_differences(O):
    """Central differences of l = sum(O * dO) with respect to each head's bias
    value equal the sum of that head's dbias over sequences and keys."""
    B, H, L, d = 2, 2, 5, 2
    seqlens = [5, 3]
    q, k, v, do = (_rand((B, H, L, d), s) for s in (63, 64, 65, 66))
    vals = np.array([-0.7, 0.2])
    for causal in (False, True):
        g = O.attention(q, k, v, seqlens, do=do, bias_mode="per_head", bias_arg=vals, causal=causal)
        eps = 1e-6
        for h in range(H):
            vp, vm = vals.copy(), vals.copy()
            vp[h] += eps
            vm[h] -= eps
            lp = np.sum(O.attention(q, k, v, seqlens, bias_mode="per_head", bias_arg=vp, causal=causal)["o"] * do)
            lm = np.sum(O.attention(q, k, v, seqlens, bias_mode="per_head", bias_arg=vm, causal=causal)["o"] * do)
            fd = (lp - lm) / (2 * eps)
            got = g["dbias"][:, h].sum()
            assert abs(fd - got) < 1e-7 * (1 + abs(fd)), (causal, h, fd, got)


def pin_per_head_matches_constant(O):
    """Head h under per-head values equals the constant-bias mode with that
    head's value, outputs and gradients (fixes which head reads which value)."""
    B, H, L, d = 2, 3, 6, 4
    seqlens = [6, 2]
    q, k, v, do = (_rand((B, H, L, d), s) for s in (67, 68, 69, 70))
    vals = np.array([0.5, -2.0, 1.25])
    g = O.attention(q, k, v, seqlens, do=do, bias_mode="per_head", bias_arg=vals)
    for h in range(H):
        c = O.attention(q, k, v, seqlens, do=do, bias_mode="const", bias_arg=float(vals[h]))
        for key in ("o", "dq", "dk", "dv", "dbias"):
            _close(g[key][:, h], c[key][:, h], what=f"per-head {key} h={h}")


ALL_PINS += [pin_dbias_zero_scores_closed_form, pin_dbias_finite_differences, pin_per_head_matches_constant]
