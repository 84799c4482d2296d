"""Checks that pin an attention implementation to facts fixed outside it.

Each check takes the implementation under test as functions
``fwd(q, k, v, scale, causal) -> (O, LSE)`` and
``bwd(q, k, v, do, scale, causal) -> (dQ, dK, dV)`` for one head, and raises
AssertionError on failure.  ``tests/test_oracle.py`` runs them on the oracle;
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with a
planted mistake and requires that some check fails.

What fixes each value:
  * closed forms of softmax attention (uniform rows when Q = 0, a single
    dominant score, N = 1);
  * invariants (row-constant shift of the scores, linearity in V, the
    identity rowsum(dO * O) = rowsum(P * dP));
  * central finite differences of L = sum(O * dO) for the gradients;
  * the values printed by the pages (golden JSON files in tests/golden/).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- forward


def check_page_cpu_vectors(fwd):
    """The page's 5x3 / 5x2 vectors: the causal first row sees only key 0, so O_0 = v_0."""
    g = load_golden("cpu_check_vectors.json")
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    o, _ = fwd(q, k, v, 1.0 / math.sqrt(3.0), True)
    np.testing.assert_allclose(o[0], g["printed"]["causal_row0_output"], atol=1e-15)


def check_zero_query(fwd, n=9, d=4, dv=3, causal=False, seed=1):
    """Q = 0 makes every visible score equal: O_i is the mean of the visible V rows
    and LSE_i = ln(number of visible keys)."""
    r = _rng(seed)
    k, v = r.standard_normal((n, d)), r.standard_normal((n, dv))
    o, lse = fwd(np.zeros((n, d)), k, v, 0.37, causal)
    for i in range(n):
        vis = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:vis].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], math.log(vis), rtol=0, atol=1e-13)


def check_dominant_score(fwd, n=8, d=5, dv=3, lam=9.0, jstar=3, causal=False, seed=2):
    """Q_i = lam*e1 for all i, K_{j*} = e1 and every other key has a zero first
    coordinate: the scores of row i are tau*lam at j* and 0 elsewhere, so
    P_{i j*} = e^{tau lam} / (e^{tau lam} + n_i - 1) and the rest is uniform."""
    r = _rng(seed)
    scale = 0.8
    q = np.zeros((n, d))
    q[:, 0] = lam
    k = r.standard_normal((n, d))
    k[:, 0] = 0.0
    k[jstar] = 0.0
    k[jstar, 0] = 1.0
    v = r.standard_normal((n, dv))
    o, lse = fwd(q, k, v, scale, causal)
    big = math.exp(scale * lam)
    for i in range(n):
        vis = list(range(i + 1)) if causal else list(range(n))
        if jstar in vis:
            others = [j for j in vis if j != jstar]
            pj = big / (big + len(others))
            expect = pj * v[jstar] + (1 - pj) * (v[others].mean(axis=0) if others else 0.0)
            expect_lse = math.log(big + len(others))
        else:
            expect = v[vis].mean(axis=0)
            expect_lse = math.log(len(vis))
        np.testing.assert_allclose(o[i], expect, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], expect_lse, rtol=0, atol=1e-12)


def check_single_key(fwd, bwd, d=6, seed=3):
    """N = 1: O = V, LSE = tau q.k, dQ = dK = 0, dV = dO."""
    r = _rng(seed)
    q, k, v, do = (r.standard_normal((1, d)) for _ in range(4))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, v, atol=1e-15)
        np.testing.assert_allclose(lse, [0.3 * float(q[0] @ k[0])], atol=1e-14)
        dq, dk, dv = bwd(q, k, v, do, 0.3, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-15)
        np.testing.assert_allclose(dk, 0.0, atol=1e-15)
        np.testing.assert_allclose(dv, do, atol=1e-15)


def check_key_shift(fwd, bwd, n=10, d=4, dv=3, causal=False, seed=4):
    """K <- K + 1 c^T adds tau q_i.c to every score of row i: O and all
    gradients are unchanged and LSE_i moves by exactly tau q_i.c."""
    r = _rng(seed)
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    v, do = r.standard_normal((n, dv)), r.standard_normal((n, dv))
    c = 3.0 * r.standard_normal(d)
    scale = 0.45
    o1, l1 = fwd(q, k, v, scale, causal)
    o2, l2 = fwd(q, k + c[None, :], v, scale, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q @ c), atol=1e-12)
    g1 = bwd(q, k, v, do, scale, causal)
    g2 = bwd(q, k + c[None, :], v, do, scale, causal)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(b, a, atol=1e-11)


def check_value_linearity(fwd, n=7, d=3, dv=4, causal=True, seed=5):
    """O is linear in V: O(aV + bV') = a O(V) + b O(V')."""
    r = _rng(seed)
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    v1, v2 = r.standard_normal((n, dv)), r.standard_normal((n, dv))
    o1, _ = fwd(q, k, v1, 0.6, causal)
    o2, _ = fwd(q, k, v2, 0.6, causal)
    o3, _ = fwd(q, k, 2.5 * v1 - 1.5 * v2, 0.6, causal)
    np.testing.assert_allclose(o3, 2.5 * o1 - 1.5 * o2, atol=1e-12)


# --------------------------------------------------------------------------- backward


def check_finite_differences(fwd, bwd, n=6, d=4, dv=3, causal=False, scale=0.7,
                             seed=6, h=1e-6, tol=1e-7):
    """Central differences of L = sum(O * dO) against the analytic dQ, dK, dV."""
    r = _rng(seed)
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    v, do = r.standard_normal((n, dv)), r.standard_normal((n, dv))

    def loss(qq, kk, vv):
        o, _ = fwd(qq, kk, vv, scale, causal)
        return float((o * do).sum())

    grads = bwd(q, k, v, do, scale, causal)
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=tol,
                                   err_msg=f"gradient {'qkv'[which]} (causal={causal})")


def check_zero_query_gradients(bwd, n=8, d=4, dv=3, causal=False, seed=7):
    """Q = 0 makes P uniform over the n_i visible keys.  Then
    dK = 0,  dV_j = sum_{i sees j} dO_i / n_i,
    dQ_i = (tau / n_i) * sum_{j visible} (dO_i . (v_j - vbar_i)) k_j."""
    r = _rng(seed)
    k, v, do = r.standard_normal((n, d)), r.standard_normal((n, dv)), r.standard_normal((n, dv))
    scale = 0.55
    dq, dk, dv_ = bwd(np.zeros((n, d)), k, v, do, scale, causal)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    exp_dv = np.zeros((n, dv))
    exp_dq = np.zeros((n, d))
    for i in range(n):
        vis = i + 1 if causal else n
        exp_dv[:vis] += do[i] / vis
        vbar = v[:vis].mean(axis=0)
        coef = (v[:vis] - vbar) @ do[i]
        exp_dq[i] = scale / vis * (coef @ k[:vis])
    np.testing.assert_allclose(dv_, exp_dv, atol=1e-13)
    np.testing.assert_allclose(dq, exp_dq, atol=1e-13)
