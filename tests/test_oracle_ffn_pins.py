"""Pins of the fp64 FFN oracle to things other than itself: brute force with
exact sums, SiLU identities against scipy, closed forms and invariants."""
import math

import numpy as np
import scipy.special

import oracle
import workloads as WL


def _bf(rng, shape, std=1.0):
    return WL.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


def test_silu_identities():
    x = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(-x), oracle.silu(x) - x, rtol=1e-12, atol=1e-12)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert oracle.silu(np.array([-800.0]))[0] == 0.0           # no overflow warning turned into a wrong value


def test_ffn_brute_force_exact_sums():
    rng = np.random.default_rng(70)
    n, d, F = 5, 8, 6
    X, Wg, Wu, Wd = _bf(rng, (n, d)), _bf(rng, (F, d), 0.5), _bf(rng, (F, d), 0.5), _bf(rng, (d, F), 0.5)
    Y, A = oracle.ffn_rows(X, Wg, Wu, Wd)
    x, wg, wu, wd = (oracle.widen_bf16(t) for t in (X, Wg, Wu, Wd))
    for i in range(n):
        a = []
        for f in range(F):
            g = math.fsum(float(x[i, k]) * float(wg[f, k]) for k in range(d))
            u = math.fsum(float(x[i, k]) * float(wu[f, k]) for k in range(d))
            a.append(g / (1.0 + math.exp(-g)) * u)
        np.testing.assert_allclose(A[i], a, rtol=1e-13, atol=1e-15)
        for j in range(d):
            y = math.fsum(a[f] * float(wd[j, f]) for f in range(F))
            assert abs(Y[i, j] - y) <= 1e-12 * max(1.0, abs(y))


def test_ffn_closed_form_single_unit():
    """F = 1 with W_gate = e_0, W_up = e_1, W_down = e_2: y_2 = SiLU(x_0) x_1, the rest 0."""
    d = 4
    X = WL.bf16_round(np.array([[1.5, -2.0, 3.0, 0.5], [-0.75, 4.0, 1.0, 2.0]], np.float32))
    eye = np.eye(d, dtype=np.float32)
    Wg, Wu = WL.bf16_round(eye[:1]), WL.bf16_round(eye[1:2])
    Wd = WL.bf16_round(eye[:, 2:3])
    Y, _ = oracle.ffn_rows(X, Wg, Wu, Wd)
    x = oracle.widen_bf16(X)
    want = np.zeros((2, d))
    want[:, 2] = x[:, 0] / (1 + np.exp(-x[:, 0])) * x[:, 1]
    np.testing.assert_allclose(Y, want, rtol=1e-15, atol=0)


def test_ffn_zero_cases_and_linearity():
    rng = np.random.default_rng(71)
    n, d, F = 6, 16, 12
    X, Wg, Wu, Wd = _bf(rng, (n, d)), _bf(rng, (F, d), 0.3), _bf(rng, (F, d), 0.3), _bf(rng, (d, F), 0.3)
    assert np.all(oracle.ffn_rows(np.zeros_like(X), Wg, Wu, Wd)[0] == 0.0)
    assert np.all(oracle.ffn_rows(X, Wg, np.zeros_like(Wu), Wd)[0] == 0.0)
    Y = oracle.ffn_rows(X, Wg, Wu, Wd)[0]
    Wd2 = WL.bf16_round(2 * oracle.widen_bf16(Wd).astype(np.float32))   # exact doubling in bf16
    np.testing.assert_allclose(oracle.ffn_rows(X, Wg, Wu, Wd2)[0], 2 * Y, rtol=1e-13, atol=1e-15)
    # swapping the rows of W_down swaps the output columns
    perm = rng.permutation(d)
    np.testing.assert_allclose(oracle.ffn_rows(X, Wg, Wu, Wd[perm])[0], Y[:, perm], rtol=1e-13, atol=1e-15)


def test_ffn_chunk_invariance_and_row_independence():
    rng = np.random.default_rng(72)
    L, d, F = 37, 16, 24
    X, Wg, Wu, Wd = _bf(rng, (L, d)), _bf(rng, (F, d), 0.3), _bf(rng, (F, d), 0.3), _bf(rng, (d, F), 0.3)
    full = oracle.ffn_rows(X, Wg, Wu, Wd)[0]
    for c in (1, 5, 16, 37, 100):
        np.testing.assert_allclose(oracle.ffn_chunked(X, Wg, Wu, Wd, c), full, rtol=1e-12, atol=1e-14)
    X2 = X.copy()
    X2[10] = _bf(rng, d)
    Y2 = oracle.ffn_rows(X2, Wg, Wu, Wd)[0]
    keep = [i for i in range(L) if i != 10]
    np.testing.assert_array_equal(Y2[keep], full[keep])


def test_ffn_bound_dominates_terms():
    rng = np.random.default_rng(73)
    X, Wg, Wu, Wd = _bf(rng, (4, 32)), _bf(rng, (20, 32), 0.2), _bf(rng, (20, 32), 0.2), _bf(rng, (32, 20), 0.2)
    Y, A, B, Q = oracle.ffn_rows(X, Wg, Wu, Wd, want_bound=True)
    assert np.all(B >= np.abs(Y) - 1e-12)
    wd = oracle.widen_bf16(Wd)
    for i in range(4):
        for j in (0, 7, 31):
            terms = [A[i, f] * wd[j, f] for f in range(20)]
            assert abs(B[i, j] - math.fsum(abs(t) for t in terms)) < 1e-12
            assert abs(Q[i, j] - math.fsum(t * t for t in terms)) < 1e-12
    assert np.all(np.sqrt(Q) <= B + 1e-12)
