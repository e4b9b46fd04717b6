"""Pins of the softmax oracle (oracle/softmax_oracle.py): facts fixed by the
definition of row-softmax attention and by calculus, checked without re-running
the oracle's own formulas.  Each pin takes the oracle module (so a mutated copy
can be checked too) and raises on failure."""
import math

import numpy as np


def _rand(seed, B, H, L, d, scale=1.0):
    r = np.random.default_rng(seed)
    return [scale * r.standard_normal((B, H, L, d)) for _ in range(4)]


def pin_unit_values_give_ones(O):
    """Each valid row of weights sums to 1, so V = 1 gives O = 1 there."""
    q, k, _, _ = _rand(1, 2, 2, 9, 4)
    v = np.ones_like(q)
    n = [9, 5]
    o = O.attention(q, k, v, n)["o"]
    for b, nb in enumerate(n):
        assert np.allclose(o[b, :, :nb], 1.0, atol=1e-13)
        assert np.all(o[b, :, nb:] == 0)


def pin_zero_query_is_mean_of_values(O):
    """Q = 0: every valid key gets weight 1/n, O_i = mean of the valid V rows,
    and the log-sum-exp of n zeros is ln n."""
    _, k, v, _ = _rand(2, 2, 3, 11, 8)
    q = np.zeros_like(k)
    n = [11, 4]
    out = O.attention(q, k, v, n)
    for b, nb in enumerate(n):
        mean = v[b, :, :nb].mean(axis=1, keepdims=True)
        assert np.allclose(out["o"][b, :, :nb], np.broadcast_to(mean, out["o"][b, :, :nb].shape), atol=1e-13)
        assert np.allclose(out["lse"][b, :, :nb], math.log(nb), atol=1e-13)


def pin_single_key(O):
    """n = 1: the only weight is 1, O_0 = v_0, lse = q.k / sqrt(d)."""
    q, k, v, _ = _rand(3, 1, 2, 4, 16)
    out = O.attention(q, k, v, [1])
    assert np.allclose(out["o"][0, :, 0], v[0, :, 0], atol=1e-14)
    assert np.allclose(out["lse"][0, :, 0], np.sum(q[0, :, 0] * k[0, :, 0], axis=-1) / 4.0, atol=1e-13)


def pin_brute_force_loops(O):
    """Scalar loops with math.exp on a tiny ragged batch, every output and lse."""
    q, k, v, _ = _rand(4, 2, 1, 5, 3, scale=1.5)
    n = [5, 3]
    out = O.attention(q, k, v, n)
    for b, nb in enumerate(n):
        for i in range(nb):
            s = [sum(q[b, 0, i, c] * k[b, 0, j, c] for c in range(3)) / math.sqrt(3) for j in range(nb)]
            z = sum(math.exp(x) for x in s)
            assert abs(out["lse"][b, 0, i] - math.log(z)) < 1e-12
            for c in range(3):
                ref = sum(math.exp(s[j]) / z * v[b, 0, j, c] for j in range(nb))
                assert abs(out["o"][b, 0, i, c] - ref) < 1e-12


def pin_finite_differences(O):
    """Central differences of l = sum(O * dO) for every input entry (h = 1e-6)."""
    q, k, v, do = _rand(5, 1, 1, 4, 3)
    n = [4]
    g = O.attention(q, k, v, n, do=do)
    h = 1e-6
    for name, x, key in (("q", q, "dq"), ("k", k, "dk"), ("v", v, "dv")):
        for idx in np.ndindex(x.shape):
            if idx[2] >= n[0]:
                continue
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            lp = np.sum(O.attention(args_p["q"], args_p["k"], args_p["v"], n)["o"] * do)
            lm = np.sum(O.attention(args_m["q"], args_m["k"], args_m["v"], n)["o"] * do)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[key][idx]) < 1e-7 * (1 + abs(fd)), (name, idx, fd, g[key][idx])


def pin_explicit_jacobian(O):
    """dQ from the explicit row Jacobian (diag(p) - p p^T) built entry by entry."""
    q, k, v, do = _rand(6, 1, 1, 4, 2)
    n = [4]
    g = O.attention(q, k, v, n, do=do)
    s = 1.0 / math.sqrt(2)
    Q, K, V, G = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    dq = np.zeros_like(Q)
    for i in range(4):
        x = [s * float(Q[i] @ K[j]) for j in range(4)]
        z = sum(math.exp(t) for t in x)
        p = [math.exp(t) / z for t in x]
        dp = [float(G[i] @ V[j]) for j in range(4)]
        for j in range(4):
            dxj = sum((p[j] * (1.0 if j == m else 0.0) - p[j] * p[m]) * dp[m] for m in range(4))
            dq[i] += s * dxj * K[j]
    assert np.allclose(g["dq"][0, 0], dq, atol=1e-12)


def pin_padding_carries_nothing(O):
    """Garbage in padded rows of Q, K, V, dO leaves every output unchanged."""
    q, k, v, do = _rand(7, 2, 2, 8, 4)
    n = [8, 3]
    a = O.attention(q, k, v, n, do=do)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[1, :, 3:] = 1e6
    b = O.attention(q2, k2, v2, n, do=do2)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def pin_key_permutation(O):
    """Permuting the valid keys (K and V together) leaves O and lse unchanged."""
    q, k, v, _ = _rand(8, 1, 2, 6, 4)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = O.attention(q, k, v, [6])
    b = O.attention(q, k[:, :, perm], v[:, :, perm], [6])
    assert np.allclose(a["o"], b["o"], atol=1e-13)
    assert np.allclose(a["lse"], b["lse"], atol=1e-13)


def pin_gradient_rows_sum(O):
    """Softmax rows sum to 1 for any scores, so sum_j dX_ij = 0: the dQ rows
    are unchanged when the same vector is added to every key row (a constant
    shift of each score row)."""
    q, k, v, do = _rand(9, 1, 1, 5, 4)
    g1 = O.attention(q, k, v, [5], do=do)
    k2 = k + np.array([0.3, -1.1, 0.7, 2.0])
    g2 = O.attention(q, k2, v, [5], do=do)
    assert np.allclose(g1["o"], g2["o"], atol=1e-12)
    assert np.allclose(g1["dq"], g2["dq"], atol=1e-12)


def pin_zero_length(O):
    q, k, v, do = _rand(10, 2, 1, 4, 2)
    out = O.attention(q, k, v, [0, 2], do=do)
    for key in out:
        assert np.all(out[key][0] == 0)


ALL_PINS = [pin_unit_values_give_ones, pin_zero_query_is_mean_of_values, pin_single_key, pin_brute_force_loops,
            pin_finite_differences, pin_explicit_jacobian, pin_padding_carries_nothing, pin_key_permutation,
            pin_gradient_rows_sum, pin_zero_length]


def pin_row_term_identity(O):
    """sum_k P_ik dP_ik = rowsum(dO_i * O_i) (O_i = sum_k P_ik V_k): the row
    term of the softmax Jacobian computed by scalar loops from the weights
    equals the one formed from the oracle's O; and the oracle's dQ row i is
    s * sum_j P_ij (dP_ij - that term) K_j, also by scalar loops."""
    q, k, v, do = _rand(11, 1, 1, 6, 4)
    out = O.attention(q, k, v, [6], do=do)
    d = 4
    for i in range(6):
        s = [sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) / math.sqrt(d) for j in range(6)]
        z = sum(math.exp(x) for x in s)
        p = [math.exp(x) / z for x in s]
        dp = [sum(do[0, 0, i, c] * v[0, 0, j, c] for c in range(d)) for j in range(6)]
        row = sum(p[j] * dp[j] for j in range(6))
        assert abs(row - float(np.sum(do[0, 0, i] * out["o"][0, 0, i]))) < 1e-12
        for c in range(d):
            ref = sum(p[j] * (dp[j] - row) * k[0, 0, j, c] for j in range(6)) / math.sqrt(d)
            assert abs(out["dq"][0, 0, i, c] - ref) < 1e-12


ALL_PINS.append(pin_row_term_identity)


def pin_causal_zero_query(O):
    """Causal, Q = 0: O_i = mean of V_0..V_i and lse_i = ln(i + 1)."""
    _, k, v, _ = _rand(12, 1, 2, 7, 3)
    q = np.zeros_like(k)
    out = O.attention(q, k, v, [7], causal=True)
    for i in range(7):
        assert np.allclose(out["o"][0, :, i], v[0, :, :i + 1].mean(axis=1), atol=1e-13)
        assert np.allclose(out["lse"][0, :, i], math.log(i + 1), atol=1e-13)


def pin_causal_prefix_and_gradients(O):
    """Rows after i cannot change O_i; central differences of the causal loss."""
    q, k, v, do = _rand(13, 1, 1, 4, 2)
    a = O.attention(q, k, v, [4], do=do, causal=True)
    k2 = k.copy()
    k2[:, :, 2:] += 5.0
    b = O.attention(q, k2, v, [4], do=do, causal=True)
    assert np.allclose(a["o"][:, :, :2], b["o"][:, :, :2], atol=1e-13)
    h = 1e-6
    for idx in np.ndindex(q.shape):
        qp, qm = q.copy(), q.copy()
        qp[idx] += h
        qm[idx] -= h
        fd = (np.sum(O.attention(qp, k, v, [4], causal=True)["o"] * do)
              - np.sum(O.attention(qm, k, v, [4], causal=True)["o"] * do)) / (2 * h)
        assert abs(fd - a["dq"][idx]) < 1e-7 * (1 + abs(fd))


ALL_PINS += [pin_causal_zero_query, pin_causal_prefix_and_gradients]
