"""Pins for the oracle's Hessian and prepare steps (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle.prepare import NotPositiveDefinite


def test_hessian_term_by_term():
    """S = sum_t x_t x_t^T, written out with scalar loops on a tiny X."""
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 5)).astype(np.float32)
    S = oracle.hessian_S([X])
    T, n = X.shape
    for i in range(n):
        for j in range(n):
            acc = 0.0
            for t in range(T):
                acc += float(X[t, i]) * float(X[t, j])
            assert abs(S[i, j] - acc) <= 1e-12 * max(1.0, abs(acc))
    assert np.array_equal(oracle.hessian([X]), 2.0 * S)


def test_hessian_symmetric_psd_and_additive():
    rng = np.random.default_rng(1)
    X1 = rng.standard_normal((30, 12))
    X2 = rng.standard_normal((9, 12))
    S = oracle.hessian_S([X1, X2])
    assert np.allclose(S, S.T, rtol=0, atol=1e-12)
    assert np.linalg.eigvalsh(S).min() > -1e-10
    assert np.allclose(S, oracle.hessian_S([np.vstack([X1, X2])]), rtol=1e-14, atol=1e-12)


def _random_S(n, tokens=None, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((tokens or 4 * n, n))
    X[:, rng.choice(n, max(1, n // 50), replace=False)] *= 20
    return oracle.hessian_S([X])


def test_prepare_factor_properties():
    S = _random_S(96)
    P = oracle.prepare(S, 0.01, False)
    U = P.U
    assert np.allclose(np.tril(U, -1), 0.0)
    assert np.all(np.diag(U) > 0)
    I = np.eye(96)
    assert np.abs(U.T @ U @ P.Hd - I).max() < 1e-10


def test_prepare_ul_route_equals_textbook_route():
    """U = R^-1 where H_d = R R^T with R upper (reverse-order Cholesky), computed with
    numpy's Cholesky on the index-reversed matrix, equals the oracle's LAPACK route."""
    S = _random_S(80, seed=3)
    P = oracle.prepare(S, 0.01, False)
    J = np.eye(80)[::-1]
    Lr = np.linalg.cholesky(J @ P.Hd @ J)  # lower
    R = J @ Lr @ J                          # upper, H_d = R R^T
    assert np.abs(R @ R.T - P.Hd).max() < 1e-9 * np.abs(P.Hd).max()
    U_ul = np.linalg.inv(R)
    assert np.abs(U_ul - P.U).max() <= 1e-12 * np.abs(P.U).max()


def test_damping_closed_form_on_diagonal_S():
    d = np.array([1.0, 4.0, 9.0, 16.0])
    P = oracle.prepare(np.diag(d), perc_damp=0.05, desc_act=False)
    lam = 0.05 * np.mean(2.0 * d)
    assert P.lam == pytest.approx(lam, rel=1e-15)
    assert np.allclose(P.U, np.diag(1.0 / np.sqrt(2.0 * d + lam)), rtol=1e-14, atol=0)


def test_dead_columns():
    S = _random_S(10, seed=5)
    S[3, :] = 0.0
    S[:, 3] = 0.0
    P = oracle.prepare(S, 0.01, False)
    assert P.dead.tolist() == [i == 3 for i in range(10)]
    assert P.H[3, 3] == 1.0


def test_desc_act_order_is_stable_descending_diagonal():
    d = np.array([2.0, 5.0, 2.0, 7.0, 5.0, 1.0])
    P = oracle.prepare(np.diag(d), 0.01, True)
    assert P.perm.tolist() == [3, 1, 4, 0, 2, 5]
    assert np.allclose(np.diag(P.H), 2.0 * d[P.perm])


def test_not_positive_definite_without_damping():
    S = np.array([[1.0, 2.0], [2.0, 1.0]])  # indefinite
    with pytest.raises(NotPositiveDefinite):
        oracle.prepare(S, 0.0, False)


def test_accepted_order_near_ties():
    d = np.array([5.0, 3.0, 3.0 + 1e-9, 1.0])
    # exact order puts index 2 before 1; swapping them is within tolerance
    assert oracle.check_descending_order(np.array([0, 1, 2, 3]), d, 1e-6) == 2
    assert oracle.check_descending_order(np.array([0, 2, 1, 3]), d, 1e-6) == 0
    with pytest.raises(ValueError):
        oracle.check_descending_order(np.array([1, 0, 2, 3]), d, 1e-6)
    with pytest.raises(ValueError):
        oracle.check_descending_order(np.array([0, 0, 2, 3]), d, 1e-6)
    P = oracle.prepare(np.diag(d), 0.01, True, order=np.array([0, 1, 2, 3]))
    assert P.perm.tolist() == [0, 1, 2, 3]
    assert np.allclose(np.diag(P.H), 2 * d)
