"""Pins of the fp64 Nystrom low-rank factor oracle (oracle/nystrom_oracle.py)
against what the Clean paper's section 2.2, section 3 and Appendix A fix
and against the mathematics: exact reconstruction of a rank-r PSD matrix,
the warm start agreeing with the cold start once the passes have converged,
Algorithm 3 reducing to Algorithm 2, the preconditioner's action on U and
on its complement, and full rank reducing to the exact-root Shampoo factor
(LAPACK eigh through the OKLS oracle).  No GPU is needed.
"""
import math

import numpy as np
import pytest

from oracle import nystrom_oracle as Y
from oracle import okls_oracle as O


def _orth(rng, m, k):
    q, r = np.linalg.qr(rng.standard_normal((m, k)))
    return q * np.sign(np.diag(r))


def _psd(rng, m, lam):
    Q = _orth(rng, m, len(lam))
    return (Q * np.asarray(lam)) @ Q.T, Q


def test_eps32_is_the_single_precision_spacing():
    for x in (1.0, 3.0, 1e-3, 12345.678, 2.0 ** 40):
        assert Y.eps32(x) == float(np.spacing(np.float32(x)))


def test_exact_rank_r_matrix_is_reproduced():
    """A PSD matrix of rank <= r lies in the span of any generic sketch of
    r + p columns, so its Nystrom approximation is exact; Algorithm 2 sketches
    the shifted A + nu I instead, whose approximation differs from it by
    O(nu), and removing the shift returns A's eigenvalues to within O(nu)
    (section 2.2, Algorithm 2).  A shift of 0 (nu = 0 by hand) is exact to
    rounding."""
    rng = np.random.default_rng(0)
    m, r, p = 60, 8, 4
    for rank in (8, 5):
        lam = np.linspace(3.0, 0.5, rank)
        A, _ = _psd(rng, m, lam)
        Psi = rng.standard_normal((m, r + p))
        U, L, nu = Y.nystrom(lambda X: A @ X, m, r, p, 0, None, Psi)
        assert nu > 0 and nu < 1e-6 * np.max(lam)
        np.testing.assert_allclose((U * L) @ U.T, A, rtol=0, atol=32 * nu)
        np.testing.assert_allclose(L[:rank], np.sort(lam)[::-1], rtol=0, atol=32 * nu)
        np.testing.assert_allclose(L[rank:], 0.0, rtol=0, atol=32 * nu)
        # eq. 4 unshifted (Y B^+ Y^T with the pseudo-inverse) is exact
        Om = Y.thin_qr(Psi)
        Yk = A @ Om
        At = Yk @ np.linalg.pinv(Om.T @ Yk) @ Yk.T
        np.testing.assert_allclose(At, A, atol=1e-10)
        np.testing.assert_allclose(U.T @ U, np.eye(r), atol=1e-12)


def test_algorithm3_without_warm_start_or_passes_is_algorithm2():
    rng = np.random.default_rng(1)
    m, r, p = 40, 6, 3
    A, _ = _psd(rng, m, np.logspace(0, -4, m))
    Psi = rng.standard_normal((m, r + p))
    U3, L3, _ = Y.nystrom(lambda X: A @ X, m, r, p, 0, None, Psi)
    U2, L2 = Y.nystrom_alg2(A, r, Psi)
    np.testing.assert_allclose(L3, L2, rtol=1e-13)
    np.testing.assert_allclose(np.abs(U3.T @ U2), np.eye(r), atol=1e-10)


def test_warm_start_agrees_with_cold_start_after_enough_passes():
    """With a spectral gap after the r-th eigenvalue, subspace iteration
    converges to the top-r eigenspace from any start: after q passes the
    warm-started and cold-started factors agree (projectors and eigenvalues)
    and both are the top-r eigenpairs of A (LAPACK eigh)."""
    rng = np.random.default_rng(2)
    m, r, p = 80, 6, 4
    lam = np.concatenate([np.linspace(2.0, 1.0, r), 1e-3 * rng.random(m - r)])
    A, _ = _psd(rng, m, lam)
    warm = _orth(rng, m, r)
    Psi = rng.standard_normal((m, r + p))
    Uc, Lc, _ = Y.nystrom(lambda X: A @ X, m, r, p, 6, None, Psi)
    Uw, Lw, _ = Y.nystrom(lambda X: A @ X, m, r, p, 6, warm, Psi)
    np.testing.assert_allclose(Uc @ Uc.T, Uw @ Uw.T, atol=1e-9)
    np.testing.assert_allclose(Lc, Lw, rtol=1e-9)
    w, E = np.linalg.eigh(A)
    np.testing.assert_allclose(Lc, w[::-1][:r], rtol=1e-9)
    Et = E[:, ::-1][:, :r]
    np.testing.assert_allclose(Uc @ Uc.T, Et @ Et.T, atol=1e-9)
    # signs follow the warm start (Algorithm 3's last line)
    assert np.all(np.sum(Uw * warm, axis=0) >= 0)


def test_sketch_through_the_stored_factors_is_eq6():
    """Eq. 8 applies beta2 U Lambda U^T + (1 - beta2) G G^T to the test
    matrix without forming it; the refresh equals the one on the dense eq. 6
    matrix."""
    rng = np.random.default_rng(3)
    m, n, r, p = 30, 20, 5, 3
    G = rng.standard_normal((m, n))
    U0 = _orth(rng, m, r)
    lam0 = np.linspace(4.0, 1.0, r)
    hp = Y.NysHyper(rank=r, oversample=p, passes=1, beta2=0.7, period=1)
    st = Y.NysState(W=np.zeros((m, n)), M=np.zeros((m, n)), UL=U0, lamL=lam0, UR=_orth(rng, n, r),
                    lamR=np.linspace(3.0, 1.0, r))
    PsiL, PsiR = rng.standard_normal((m, r + p)), rng.standard_normal((n, r + p))
    res = Y.nys_step(st, G, hp, 1, PsiL, PsiR)
    Ad = 0.7 * (U0 * lam0) @ U0.T + 0.3 * G @ G.T
    U, L, _ = Y.nystrom(lambda X: Ad @ X, m, r, p, 1, U0, PsiL)
    np.testing.assert_allclose(res.state.UL, U, atol=1e-12)
    np.testing.assert_allclose(res.state.lamL, L, rtol=1e-12)


def test_preconditioner_on_u_and_its_complement():
    """Eq. 5/9: P^-1/2 scales u_i by sqrt((lambda_r + mu) / (lambda_i + mu))
    and is the identity on the orthogonal complement of U."""
    rng = np.random.default_rng(4)
    d, r, mu = 25, 6, 1e-3
    U = _orth(rng, d, r)
    lam = np.linspace(5.0, 0.2, r)
    P = Y.inv_sqrt_precond(U, lam, mu, d)
    np.testing.assert_allclose(P @ U, U * np.sqrt((lam[-1] + mu) / (lam + mu)), atol=1e-13)
    x = rng.standard_normal(d)
    x -= U @ (U.T @ x)
    np.testing.assert_allclose(P @ x, x, atol=1e-13)


def test_full_rank_is_the_exact_root():
    """With r = d the Nystrom factor is A itself (for d <= r + p) and
    P^-1/2 = sqrt(lambda_r + mu) (A + mu I)^-1/2, the exact-root factor of
    the OKLS oracle (LAPACK eigh); the preconditioned matrix is the exact
    Shampoo whitening up to the two constants."""
    rng = np.random.default_rng(5)
    m, n, mu = 12, 9, 1e-2
    G = rng.standard_normal((m, n))
    L, R = G @ G.T, G.T @ G
    UL, lamL, _ = Y.nystrom(lambda X: L @ X, m, m, 0, 0, None, rng.standard_normal((m, m)))
    UR, lamR, _ = Y.nystrom(lambda X: R @ X, n, n, 0, 0, None, rng.standard_normal((n, n)))
    PL = Y.inv_sqrt_precond(UL, lamL, mu, m)
    root, _ = O.inv_root_exact(L + mu * np.eye(m), 2)
    np.testing.assert_allclose(PL, math.sqrt(lamL[-1] + mu) * root, atol=1e-9)
    N = rng.standard_normal((m, n))
    Ur, _ = O.inv_root_exact(R + mu * np.eye(n), 2)
    want = math.sqrt(lamL[-1] + mu) * math.sqrt(lamR[-1] + mu) * root @ N @ Ur
    np.testing.assert_allclose(Y.precondition(UL, lamL, UR, lamR, N, mu), want, atol=1e-9)


def test_step_schedule_and_update_form():
    """Refreshes on t = 1, 1 + T, ... (Algorithm 1's first line) and the
    factors are kept bitwise in between; the update is the OKLS form with the
    momentum of the OKLS oracle; a zero gradient at the first refresh gives
    empty eigenvalues and a pure decay (N8)."""
    rng = np.random.default_rng(6)
    m, n = 24, 16
    hp = Y.NysHyper(rank=4, oversample=2, passes=1, period=3, lr=0.05)
    st = Y.init_state(rng.standard_normal((m, n)))
    seen = []
    for t in range(1, 8):
        G = rng.standard_normal((m, n))
        r = Y.nys_step(st, G, hp, t, rng.standard_normal((m, 6)), rng.standard_normal((n, 6)))
        seen.append(r.nu != (0.0, 0.0))
        if t not in (1, 4, 7):
            assert np.array_equal(r.state.UL, st.UL) and np.array_equal(r.state.lamR, st.lamR)
        M, N = O.momentum(st.M, G, hp.beta1, t, True)
        np.testing.assert_array_equal(r.N, N)
        U = Y.precondition(r.state.UL, r.state.lamL, r.state.UR, r.state.lamR, N, hp.eps)
        decay = 1.0 - hp.lr * hp.weight_decay
        np.testing.assert_allclose(r.state.W, decay * st.W - hp.lr * O.c_shape(m, n) * U, atol=1e-12)
        st = r.state
    assert seen == [True, False, False, True, False, False, True]
    z = Y.nys_step(Y.init_state(np.ones((m, n))), np.zeros((m, n)), hp, 1, rng.standard_normal((m, 6)),
                   rng.standard_normal((n, 6)))
    assert np.all(z.state.lamL == 0) and np.all(np.isfinite(z.state.UL))
    np.testing.assert_allclose(z.state.W, (1.0 - hp.lr * hp.weight_decay) * np.ones((m, n)), rtol=1e-15)


def test_small_sides_sketch_the_whole_space():
    """N7: a side below r + p sketches with all its columns and keeps
    min(r, d) eigenpairs; with d <= r the factor is exact."""
    rng = np.random.default_rng(7)
    d, r, p = 5, 8, 4
    A, _ = _psd(rng, d, [3.0, 2.0, 1.0, 0.5, 0.25])
    U, L, _ = Y.nystrom(lambda X: A @ X, d, r, p, 1, None, rng.standard_normal((d, r + p)))
    assert U.shape == (d, d)
    np.testing.assert_allclose((U * L) @ U.T, A, atol=1e-12)
