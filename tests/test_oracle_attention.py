"""Pins of the attention oracle (oracle/attention.py): a brute force written with scalar loops on
tiny inputs, closed forms (zero queries average the visible values; the first row of a sequence
copies its value), invariants (causality, independent sequences, a key shift moves only the
log-sum-exp, grouped heads equal repeated heads, saturation at large scores), and central
finite differences of the backward."""

import math

import numpy as np

from oracle import attention as att


def _rand(rng, T, w, scale=1.0):
    return rng.normal(size=(T, w)) * scale


def _brute(q, k, v, n_seq, n_q, n_kv, d):
    """O and lse with explicit loops over rows, keys and head dimensions (math.exp/log only)."""
    T = len(q)
    S = T // n_seq
    O = [[0.0] * (n_q * d) for _ in range(T)]
    L = [[0.0] * n_q for _ in range(T)]
    for b in range(n_seq):
        for h in range(n_q):
            g = h // (n_q // n_kv)
            for i in range(S):
                ti = b * S + i
                sc = []
                for j in range(i + 1):
                    tj = b * S + j
                    dot = 0.0
                    for e in range(d):
                        dot += q[ti][h * d + e] * k[tj][g * d + e]
                    sc.append(dot / math.sqrt(d))
                m = max(sc)
                z = sum(math.exp(x - m) for x in sc)
                L[ti][h] = m + math.log(z)
                for e in range(d):
                    O[ti][h * d + e] = sum(math.exp(sc[j] - m) / z * v[b * S + j][g * d + e] for j in range(i + 1))
    return np.array(O), np.array(L)


def test_matches_brute_force_loops():
    rng = np.random.default_rng(1)
    n_seq, S, n_q, n_kv, d = 2, 5, 4, 2, 3
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), n_seq, n_q, n_kv, d)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-14)


def test_zero_queries_average_the_visible_values():
    rng = np.random.default_rng(2)
    n_seq, S, n_q, n_kv, d = 3, 7, 2, 1, 4
    T = n_seq * S
    q = np.zeros((T, n_q * d))
    k, v = _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    for b in range(n_seq):
        for i in range(S):
            t = b * S + i
            want = v[b * S: t + 1].mean(axis=0)
            for h in range(n_q):
                np.testing.assert_allclose(O[t, h * d:(h + 1) * d], want, rtol=1e-13, atol=1e-15)
                assert abs(L[t, h] - math.log(i + 1)) < 1e-13


def test_first_row_of_each_sequence_copies_its_value():
    rng = np.random.default_rng(3)
    n_seq, S, n_q, n_kv, d = 4, 3, 2, 2, 8
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    for b in range(n_seq):
        t = b * S
        np.testing.assert_array_equal(O[t], v[t])
        for h in range(n_q):
            assert abs(L[t, h] - q[t, h * d:(h + 1) * d] @ k[t, h * d:(h + 1) * d] / math.sqrt(d)) < 1e-13


def test_causal_and_sequences_independent():
    rng = np.random.default_rng(4)
    n_seq, S, n_q, n_kv, d = 2, 9, 2, 1, 4
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    O, _ = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    t = 4                      # change keys and values after row t of sequence 0, and all of sequence 1
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] += 5.0
    v2[t + 1:] -= 3.0
    O2, _ = att.forward(q, k2, v2, n_seq, n_q, n_kv, d)
    np.testing.assert_array_equal(O2[: t + 1], O[: t + 1])
    assert np.abs(O2[t + 1: S] - O[t + 1: S]).max() > 1e-3
    # sequence 0 unchanged when only sequence 1 changes
    k3 = k.copy()
    k3[S:] = rng.normal(size=k3[S:].shape)
    O3, _ = att.forward(q, k3, v, n_seq, n_q, n_kv, d)
    np.testing.assert_array_equal(O3[:S], O[:S])


def test_key_shift_moves_only_the_log_sum_exp():
    rng = np.random.default_rng(5)
    n_seq, S, n_q, n_kv, d = 2, 6, 2, 2, 4
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    u = rng.normal(size=n_kv * d)
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    O2, L2 = att.forward(q, k + u[None, :], v, n_seq, n_q, n_kv, d)
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-12)
    shift = np.stack([q[:, h * d:(h + 1) * d] @ u[h * d:(h + 1) * d] for h in range(n_q)], axis=1) / math.sqrt(d)
    np.testing.assert_allclose(L2 - L, shift, rtol=1e-10, atol=1e-11)


def test_grouped_heads_equal_repeated_heads():
    rng = np.random.default_rng(6)
    n_seq, S, n_q, n_kv, d = 2, 5, 6, 2, 4
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    grp = n_q // n_kv
    rep = lambda x: np.concatenate([x[:, (h // grp) * d:(h // grp + 1) * d] for h in range(n_q)], axis=1)  # noqa: E731
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    O2, L2 = att.forward(q, rep(k), rep(v), n_seq, n_q, n_q, d)
    np.testing.assert_allclose(O, O2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L, L2, rtol=1e-13, atol=1e-15)
    dO = _rand(rng, T, n_q * d)
    dq, dk, dv = att.backward(q, k, v, dO, n_seq, n_q, n_kv, d)
    dq2, dk2, dv2 = att.backward(q, rep(k), rep(v), dO, n_seq, n_q, n_q, d)
    np.testing.assert_allclose(dq, dq2, rtol=1e-12, atol=1e-14)
    fold = lambda x: np.concatenate([sum(x[:, h * d:(h + 1) * d] for h in range(g * grp, (g + 1) * grp))  # noqa: E731
                                     for g in range(n_kv)], axis=1)
    np.testing.assert_allclose(dk, fold(dk2), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dv, fold(dv2), rtol=1e-12, atol=1e-14)


def test_large_scores_saturate_without_overflow():
    n_seq, S, n_q, n_kv, d = 1, 4, 1, 1, 2
    q = np.array([[1.0, 0.0]] * S) * 1e4
    k = np.array([[1.0, 0.0], [3.0, 0.0], [2.0, 0.0], [-1.0, 0.0]])
    v = np.arange(8, dtype=np.float64).reshape(4, 2)
    O, L = att.forward(q, k, v, n_seq, n_q, n_kv, d)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    np.testing.assert_array_equal(O[1:], v[[1, 1, 1]])     # the largest visible key wins outright


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(7)
    n_seq, S, n_q, n_kv, d = 2, 4, 4, 2, 3
    T = n_seq * S
    q, k, v = _rand(rng, T, n_q * d), _rand(rng, T, n_kv * d), _rand(rng, T, n_kv * d)
    W = _rand(rng, T, n_q * d)
    dq, dk, dv = att.backward(q, k, v, W, n_seq, n_q, n_kv, d)

    def loss(q_, k_, v_):
        return float((att.forward(q_, k_, v_, n_seq, n_q, n_kv, d)[0] * W).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            e = np.zeros_like(x)
            e[idx] = eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name] = x + e
            args_m[name] = x - e
            fd[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                       loss(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_of_values_is_linear_and_exact():
    """O is linear in v, so dv = P^T dO exactly: check it against the forward with unit values."""
    rng = np.random.default_rng(8)
    n_seq, S, n_q, n_kv, d = 1, 5, 1, 1, 5
    q, k = _rand(rng, S, d), _rand(rng, S, d)
    dO = _rand(rng, S, d)
    _, _, dv = att.backward(q, k, np.zeros((S, d)), dO, n_seq, n_q, n_kv, d)
    # P from the forward with v = identity rows (d = S): O = P
    P, _ = att.forward(q, k, np.eye(S), n_seq, n_q, n_kv, d)
    np.testing.assert_allclose(dv, P.T @ dO, rtol=1e-13, atol=1e-15)
