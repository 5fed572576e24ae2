"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names what it pins: values printed on the pages (fixtures under
tests/golden/), closed forms, special cases that reduce to a textbook or a
library routine other than the one the oracle uses, invariants, and brute
force on tiny inputs.  No GPU is needed.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import okls_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _spd(rng, d, kappa):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.logspace(0, -math.log10(kappa), d)
    return (Q * lam) @ Q.T


def _orth(rng, d):
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    return Q * np.sign(np.diag(R))


# --------------------------------------------------------------------------
# Worked example and problem 14 of the Shampoo chapter (printed values).
# --------------------------------------------------------------------------
def test_worked_example_factor_and_singular_values():
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    eps = 1e-12
    m, n = G.shape
    Sa, Sb = O.factor_update_shampoo(eps * np.eye(m), eps * np.eye(n), G, eps)
    np.testing.assert_allclose(Sa, g["L_equals_G_GT"], atol=1e-9)
    assert Sa.size + Sb.size == g["entries_kronecker_vs_fisher_block"]["factors"]
    assert (m * n) ** 2 == g["entries_kronecker_vs_fisher_block"]["fisher_block"]
    np.testing.assert_allclose(np.linalg.svd(G, compute_uv=False), g["singular_values_G"],
                               atol=g["printed_precision"])
    tol = 1e-6
    for k, key in [(1, "singular_values_preconditioned_one_accumulation"),
                   (4, "singular_values_after_4_identical_accumulations"),
                   (100, "singular_values_after_100_identical_accumulations")]:
        Sa, Sb = eps * np.eye(m), eps * np.eye(n)
        for _ in range(k):
            Sa, Sb = O.factor_update_shampoo(Sa, Sb, G, eps)
        Pa, _ = O.inv_root_exact(Sa, 4)
        Pb, _ = O.inv_root_exact(Sb, 4)
        sv = np.linalg.svd(Pa @ G @ Pb, compute_uv=False)
        np.testing.assert_allclose(sv, g[key], atol=tol)


def test_worked_example_through_newton_schulz_quarter_root():
    """The coupled NS chain (two inverse-square-root chains) reproduces the
    printed 1, 1 / 0.5 / 0.1: G has no component in R's null space and the
    iteration maps eigen-directions to themselves."""
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    eps = 1e-9
    coeffs, _ = O.ns_coefficients(1e-3, 10)
    for k, key in [(1, "singular_values_preconditioned_one_accumulation"),
                   (4, "singular_values_after_4_identical_accumulations"),
                   (100, "singular_values_after_100_identical_accumulations")]:
        Sa, Sb = eps * np.eye(2), eps * np.eye(3)
        for _ in range(k):
            Sa, Sb = O.factor_update_shampoo(Sa, Sb, G, eps)
        sv = np.linalg.svd(O.ns_inv_quarter(Sa, coeffs) @ G @ O.ns_inv_quarter(Sb, coeffs),
                           compute_uv=False)
        np.testing.assert_allclose(sv, g[key], rtol=1e-4)


def test_worked_example_full_shampoo_step_first_update():
    """At t=1 the Nesterov reading gives N = G, so the Shampoo-mode whitened
    update is exactly L^{-1/4} G R^{-1/4}: singular values 1, 1."""
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    hp = O.Hyper(eps=1e-12)
    st = O.init_state(np.zeros_like(G), hp.eps)
    r = O.shampoo_step(st, G, hp, 1)
    np.testing.assert_allclose(r.N, G, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.svd(r.U, compute_uv=False), [1.0, 1.0], atol=1e-6)


def test_refresh_period_worked_example():
    """Roots refreshed every 3 steps on the worked example's fixed G (Shampoo
    sums): the factor accumulates every step, but P_a G P_b keeps the
    singular values of the last refresh, r^{-1/2} after r accumulations --
    1 at t = 1..3 and 0.5 at t = 4..6 (the page's value for four
    accumulations), then 1/sqrt(7)."""
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    hp = O.Hyper(eps=1e-12, root_period=3)
    st = O.init_state(np.zeros_like(G), hp.eps)
    for t in range(1, 8):
        r = O.shampoo_step(st, G, hp, t)
        st = r.state
        last = 1 + 3 * ((t - 1) // 3)
        sv = np.linalg.svd(st.Pa @ G @ st.Pb, compute_uv=False)
        np.testing.assert_allclose(sv, [last ** -0.5] * 2, atol=1e-6)
        np.testing.assert_allclose(st.Sa, t * (G @ G.T) + (t + 1) * hp.eps * np.eye(2), rtol=1e-12)
    assert abs(0.5 - 4 ** -0.5) < 1e-15 and abs(g["singular_values_after_4_identical_accumulations"][0] - 0.5) < 1e-3


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
def test_refresh_period_keeps_roots_and_updates_factors(mode):
    """A non-refresh step is a full step with the previous roots: the factors,
    momentum, whitening and update are unchanged in form; period 1 is the
    default every-step refresh."""
    rng = np.random.default_rng(41)
    m, n = 7, 5
    st = O.init_state(rng.standard_normal((m, n)), 1e-9)
    hp1, hp2 = O.Hyper(), O.Hyper(root_period=2)
    for t in (1, 2, 3):
        G = rng.standard_normal((m, n))
        r1 = O.step(st, G, hp1, t, mode, "exact")
        r2 = O.step(st, G, hp2, t, mode, "exact")
        np.testing.assert_array_equal(r1.state.Sa, r2.state.Sa)
        np.testing.assert_array_equal(r1.state.M, r2.state.M)
        if t == 2:
            np.testing.assert_array_equal(r2.state.Pa, st.Pa)
            np.testing.assert_array_equal(r2.state.Pb, st.Pb)
            np.testing.assert_allclose(r2.U, st.Pa @ r2.N @ st.Pb, rtol=1e-12)
        else:
            np.testing.assert_array_equal(r1.state.Pa, r2.state.Pa)
        st = r2.state


def test_problem14_exponent_and_scale():
    g = _gold("shampoo_problem14_scale.json")
    G = np.array(g["G"], dtype=np.float64)
    eps = 1e-12
    rtol = g["printed_precision_relative"]

    def sv(Gs, p):
        Sa, Sb = O.factor_update_shampoo(eps * np.eye(2), eps * np.eye(3), Gs, eps)
        Pa, _ = O.inv_root_exact(Sa, p)
        Pb, _ = O.inv_root_exact(Sb, p)
        return np.linalg.svd(Pa @ Gs @ Pb, compute_uv=False)

    np.testing.assert_allclose(sv(G, 4), g["quarter_root_sv_G"], atol=1e-6)
    np.testing.assert_allclose(sv(10 * G, 4), g["quarter_root_sv_10G"], atol=1e-6)
    np.testing.assert_allclose(sv(G, 2), g["half_root_sv_G"], rtol=rtol)
    np.testing.assert_allclose(sv(10 * G, 2), g["half_root_sv_10G"], rtol=rtol)


# --------------------------------------------------------------------------
# c_shape: closed forms and the Marchenko-Pastur property of the init section.
# --------------------------------------------------------------------------
def test_c_shape_closed_forms():
    for n in (16, 1024, 4096):
        assert O.c_shape(n, n) == pytest.approx(1.0 / (2.0 * math.sqrt(n)), rel=1e-15)
    assert O.c_shape(1024, 1024) == 1.0 / 64.0
    # not symmetric in (m, n): c(n, m) / c(m, n) = n / m
    assert O.c_shape(256, 128) / O.c_shape(128, 256) == pytest.approx(2.0, rel=1e-14)


def test_c_shape_orientation_marchenko_pastur():
    """The weight-initialisation section: an i.i.d. unit Gaussian (n_out x n_in)
    matrix has spectral norm near sqrt(n_in) + sqrt(n_out), so c_shape times
    it has spectral norm near sqrt(m/n) with m = rows = n_out (reading R3)."""
    rng = np.random.default_rng(3)
    for m, n in [(512, 128), (128, 512)]:
        G = rng.standard_normal((m, n))
        s = np.linalg.norm(O.c_shape(m, n) * G, 2)
        assert s == pytest.approx(math.sqrt(m / n), rel=0.05)


# --------------------------------------------------------------------------
# Exact inverse roots.
# --------------------------------------------------------------------------
def test_inv_sqrt_identity_P_S_P():
    rng = np.random.default_rng(0)
    for kappa in (1e1, 1e4, 1e8):
        S = _spd(rng, 40, kappa)
        P, k = O.inv_root_exact(S, 2)
        assert k == pytest.approx(kappa, rel=1e-6)
        np.testing.assert_allclose(P @ S @ P, np.eye(40), atol=1e-12 * kappa)


def test_inv_root_2x2_closed_form():
    """sqrt(A) = (A + sqrt(det A) I) / sqrt(tr A + 2 sqrt(det A)) for 2x2 SPD A."""
    rng = np.random.default_rng(1)
    for _ in range(20):
        B = rng.standard_normal((2, 2))
        A = B @ B.T + 0.1 * np.eye(2)
        sd = math.sqrt(np.linalg.det(A))
        R = (A + sd * np.eye(2)) / math.sqrt(np.trace(A) + 2.0 * sd)
        np.testing.assert_allclose(O.inv_root_exact(A, 2)[0], np.linalg.inv(R), rtol=1e-10)
        sd2 = math.sqrt(np.linalg.det(R))
        R2 = (R + sd2 * np.eye(2)) / math.sqrt(np.trace(R) + 2.0 * sd2)
        np.testing.assert_allclose(O.inv_root_exact(A, 4)[0], np.linalg.inv(R2), rtol=1e-10)


def test_inv_root_3x3_against_schur_sqrtm():
    rng = np.random.default_rng(2)
    for _ in range(20):
        B = rng.standard_normal((3, 3))
        A = B @ B.T + 0.05 * np.eye(3)
        R = np.real(scipy.linalg.sqrtm(A))
        np.testing.assert_allclose(O.inv_root_exact(A, 2)[0], np.linalg.inv(R), rtol=1e-9)
        R2 = np.real(scipy.linalg.sqrtm(R))
        np.testing.assert_allclose(O.inv_root_exact(A, 4)[0], np.linalg.inv(R2), rtol=1e-9)


# --------------------------------------------------------------------------
# Newton-Schulz coefficients and iteration.
# --------------------------------------------------------------------------
def test_ns_coefficients_classical_limit():
    """On a degenerate interval [1, 1] the minimax cubic is the textbook
    Newton-Schulz step (3/2, -1/2)."""
    a, b, e = O._minimax_cubic(1.0, 1.0)
    assert a == pytest.approx(1.5, abs=1e-15)
    assert b == pytest.approx(-0.5, abs=1e-15)
    assert e == pytest.approx(0.0, abs=1e-15)


def test_ns_coefficients_equioscillation_and_optimality():
    rng = np.random.default_rng(5)
    for lo in (1e-3, 0.05, 0.5, 0.9):
        a, b, e = O._minimax_cubic(lo, 1.0)
        xs = math.sqrt(-a / (3.0 * b))
        p = lambda x: x * (a + b * x * x)
        assert p(lo) - 1 == pytest.approx(-e, abs=1e-12)
        assert p(xs) - 1 == pytest.approx(e, abs=1e-12)
        assert p(1.0) - 1 == pytest.approx(-e, abs=1e-12)
        grid = np.linspace(lo, 1.0, 20001)
        err = np.max(np.abs(grid * (a + b * grid ** 2) - 1))
        assert err == pytest.approx(e, rel=1e-6)
        # no nearby (a, b) does better on the grid
        for _ in range(200):
            da, db = rng.standard_normal(2) * 1e-3 * max(abs(a), 1)
            e2 = np.max(np.abs(grid * ((a + da) + (b + db) * grid ** 2) - 1))
            assert e2 >= err - 1e-12


def test_ns_coefficients_cover_interval_and_stay_below_one():
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    assert len(coeffs) == 10
    s = np.geomspace(1e-3, 1.0, 4001)
    for k, (a, b) in enumerate(coeffs):
        s = s * (a + b * s * s)
        if k < 9:
            assert s.max() <= 1.0 + 1e-12      # per-step scale keeps iterates <= 1
    assert np.max(np.abs(s - 1.0)) <= efin * (1 + 1e-9)
    assert efin < 1e-5


def test_ns_diagonal_reduces_to_scalar_recurrences():
    rng = np.random.default_rng(7)
    lam = np.geomspace(1e-4, 3.0, 17)
    rng.shuffle(lam)
    S = np.diag(lam)
    coeffs, _ = O.ns_coefficients(1e-3, 10)
    P, R = O.ns_inv_sqrt(S, coeffs)
    c = math.sqrt(float(np.sum(lam ** 2)))
    expect = []
    for x in lam:
        s = math.sqrt(x / c)
        for a, b in coeffs:
            s = s * (a + b * s * s)
        expect.append(s / math.sqrt(x))
    np.testing.assert_allclose(np.diag(P), expect, rtol=1e-12)
    assert np.max(np.abs(P - np.diag(np.diag(P)))) == 0.0


def test_ns_matrix_iteration_matches_eigen_closed_form_and_exact_root():
    rng = np.random.default_rng(8)
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    for kappa in (1e1, 1e3, 1e5):
        S = _spd(rng, 64, kappa) * 0.37
        P, _ = O.ns_inv_sqrt(S, coeffs)
        Pc = O.ns_eigen_closed_form(S, coeffs)
        assert O.rel_frob(P, Pc) < 1e-11 * kappa ** 0.5
        Pex, _ = O.inv_root_exact(S, 2)
        # inside the design interval each eigenvalue is within the final error bound
        assert O.rel_frob(P, Pex) < 2 * efin


def test_ns_damped_matches_shifted_exact_root():
    """With damping nu the iteration converges to (S + (nu/sqrt d)||S||_F I)^{-1/2}
    (eigh of the explicitly shifted matrix), within the coefficient bound."""
    rng = np.random.default_rng(17)
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    for d, nu in [(32, 5e-3), (96, 4e-4)]:
        S = _spd(rng, d, 1e9) * 3.0           # far beyond the undamped design range
        shift = nu / math.sqrt(d) * np.linalg.norm(S)
        Pd, _ = O.inv_root_exact(S + shift * np.eye(d), 2)
        P, R = O.ns_inv_sqrt(S, coeffs, nu)
        assert O.rel_frob(P, Pd) < 2 * efin
        Rd = np.real(scipy.linalg.sqrtm(S + shift * np.eye(d)))
        assert O.rel_frob(R, Rd) < 2 * efin


@pytest.mark.parametrize("p,nu", [(2, 5e-3), (2, 2e-3), (4, 5e-3), (4, 0.0)])
def test_ns_spectral_closed_form_matches_matrix_iteration(p, nu):
    """The per-eigenvalue closed form of the damped iteration equals the fp64
    matrix iteration (one chain for p = 2, two chained on sym(R) for p = 4)
    on random SPD factors up to rounding."""
    rng = np.random.default_rng(31 + p)
    coeffs, _ = O.ns_coefficients(1e-3, 10)
    for d, kappa in ((40, 1e2), (72, 1e4)):
        S = _spd(rng, d, kappa) * 2.3e-5
        P_iter = O.ns_inv_sqrt(S, coeffs, nu)[0] if p == 2 else O.ns_inv_quarter(S, coeffs, nu)
        P_cf = O.ns_eigen_closed_form(S, coeffs, p, nu)
        assert O.rel_frob(P_iter, P_cf) < 1e-10, (d, kappa)


def test_ns_spectral_within_coefficient_bound_of_shifted_root():
    """Inside the design interval (sqrt(y) >= floor) the closed form is within
    the final minimax error of (lambda + delta c)^{-1/2}, the eigh root of the
    explicitly shifted factor; p = 4 composes two such maps."""
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    rng = np.random.default_rng(5)
    lam = np.exp(rng.uniform(np.log(1e-4), 0.0, size=500))
    nu = 5e-3
    shift = nu / math.sqrt(lam.size) * np.linalg.norm(lam)
    f = O.ns_spectral(lam, coeffs, nu, 2)
    np.testing.assert_array_less(np.abs(f * np.sqrt(lam + shift) - 1.0), efin * (1 + 1e-9))
    # p = 4: the second chain takes the square root of R = (S + shift)^{-1/2}
    # shifted by its own nu / sqrt(d) ||R||_F; each chain contributes at most
    # efin (the first one's relative error halves under the square root)
    r = 1.0 / np.sqrt(lam + shift)
    shift2 = nu / math.sqrt(lam.size) * np.linalg.norm(r)
    f4 = O.ns_spectral(lam, coeffs, nu, 4)
    np.testing.assert_array_less(np.abs(f4 / np.sqrt(r + shift2) - 1.0), 2.5 * efin)


def test_ns_spectral_zero_eigenvalue_is_the_iteration_limit():
    """A rank-deficient factor: in a zero eigen-direction Z Y stays 0, so each
    T_k acts there as a_k and P = prod(a_k) / sqrt(c').  The closed form gives
    that value, also for an eigenvalue rounded below zero, and matches the
    matrix iteration on a singular PSD matrix."""
    coeffs, _ = O.ns_coefficients(1e-3, 10)
    lam = np.array([-1e-18, 0.0, 0.25, 1.0])
    f = O.ns_spectral(lam, coeffs, 0.0, 2)
    want0 = np.prod([a for a, _ in coeffs]) / math.sqrt(np.linalg.norm(lam))
    np.testing.assert_allclose(f[:2], want0, rtol=1e-12)
    assert np.all(np.isfinite(O.ns_spectral(lam, coeffs, 0.0, 4)))
    rng = np.random.default_rng(11)
    V, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    S = (V * np.array([0.0, 0.0, 1e-2, 0.1, 0.5, 1.0])) @ V.T
    P, _ = O.ns_inv_sqrt(S, coeffs)
    np.testing.assert_allclose(O.ns_eigen_closed_form(S, coeffs), P, rtol=1e-9, atol=1e-9)


def test_ns_damped_isotropic():
    """S = s I: ||S||_F = s sqrt(d), so the shifted matrix is s (1 + nu) I."""
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    for s, nu, d in [(1e-6, 5e-3, 16), (7.0, 0.2, 9)]:
        P, _ = O.ns_inv_sqrt(s * np.eye(d), coeffs, nu)
        np.testing.assert_allclose(P, np.eye(d) / math.sqrt(s * (1 + nu)), rtol=2 * efin)


def test_ns_isotropic():
    coeffs, efin = O.ns_coefficients(1e-3, 10)
    for s in (1e-6, 1.0, 5e3):
        P, _ = O.ns_inv_sqrt(s * np.eye(9), coeffs)
        np.testing.assert_allclose(P, np.eye(9) / math.sqrt(s), rtol=2 * efin)


# --------------------------------------------------------------------------
# Momentum with the variance-correction reading.
# --------------------------------------------------------------------------
def test_first_step_momentum_is_gradient():
    rng = np.random.default_rng(9)
    G = rng.standard_normal((5, 7))
    M, N = O.momentum(np.zeros_like(G), G, 0.9684, 1)
    np.testing.assert_allclose(N, G, rtol=1e-14)
    np.testing.assert_allclose(M, (1 - 0.9684) * G, rtol=1e-14)


def test_nesterov_output_has_unit_rms_monte_carlo():
    """For independent unit-variance gradients the corrected Nesterov output has
    unit variance at every step (what the correction is read to mean)."""
    rng = np.random.default_rng(10)
    beta1 = 0.9684
    n_series, T = 200000, 40
    M = np.zeros(n_series)
    for t in range(1, T + 1):
        G = rng.standard_normal(n_series)
        M, N = O.momentum(M, G, beta1, t)
        if t in (1, 2, 5, 20, 40):
            assert np.var(N) == pytest.approx(1.0, rel=0.02)


# --------------------------------------------------------------------------
# Factor update normalisation, whole-step invariants, update closed form.
# --------------------------------------------------------------------------
def test_okls_factor_expectation_is_per_entry_second_moment():
    """With P = I and white unit gradients, (1-beta2)/n G G^T and
    (1-beta2)/m G^T G both have expectation (1-beta2) I: the 1/n and 1/m
    normalise the sum over the other axis (catches a swapped normaliser)."""
    rng = np.random.default_rng(11)
    m, n, beta2, K = 6, 11, 0.9482, 4000
    acc_a, acc_b = np.zeros((m, m)), np.zeros((n, n))
    for _ in range(K):
        G = rng.standard_normal((m, n))
        Sa, Sb = O.factor_update_okls(np.zeros((m, m)), np.zeros((n, n)), np.eye(m), np.eye(n), G, beta2, 0.0)
        acc_a += Sa
        acc_b += Sb
    np.testing.assert_allclose(acc_a / K, (1 - beta2) * np.eye(m), atol=0.1 * (1 - beta2))
    np.testing.assert_allclose(acc_b / K, (1 - beta2) * np.eye(n), atol=0.1 * (1 - beta2))


def test_okls_factor_update_brute_force_outer_products():
    """Tiny case, explicit sums of outer products of the rows/columns of the
    cross-preconditioned gradients."""
    rng = np.random.default_rng(12)
    m, n = 3, 4
    G = rng.standard_normal((m, n))
    Pa = _spd(rng, m, 10.0)
    Pb = _spd(rng, n, 10.0)
    Sa0 = _spd(rng, m, 5.0)
    Sb0 = _spd(rng, n, 5.0)
    beta2, eps = 0.9, 1e-3
    Sa, Sb = O.factor_update_okls(Sa0, Sb0, Pa, Pb, G, beta2, eps)
    ea = beta2 * Sa0 + eps * np.eye(m)
    for j in range(n):      # columns of X_a = G P_b
        col = np.array([sum(G[i, k] * Pb[k, j] for k in range(n)) for i in range(m)])
        ea += (1 - beta2) / n * np.outer(col, col)
    eb = beta2 * Sb0 + eps * np.eye(n)
    for i in range(m):      # rows of X_b = P_a G
        row = np.array([sum(Pa[i, k] * G[k, j] for k in range(m)) for j in range(n)])
        eb += (1 - beta2) / m * np.outer(row, row)
    np.testing.assert_allclose(Sa, ea, rtol=1e-13)
    np.testing.assert_allclose(Sb, eb, rtol=1e-13)


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
def test_factor_block_is_principal_submatrix_of_full_update(mode):
    """The sampled factor update (rows of X, principal block) equals the same
    block of the full update, on both sides."""
    rng = np.random.default_rng(12)
    m, n = 23, 31
    G = rng.standard_normal((m, n))
    Sa, Sb = _spd(rng, m, 10.0), _spd(rng, n, 10.0)
    Pa, Pb = _spd(rng, m, 5.0), _spd(rng, n, 5.0)
    if mode == "okls":
        Sa2, Sb2 = O.factor_update_okls(Sa, Sb, Pa, Pb, G, 0.9482, 1e-9)
    else:
        Sa2, Sb2 = O.factor_update_shampoo(Sa, Sb, G, 1e-9)
    for side, S, S2, den, d in (("a", Sa, Sa2, n, m), ("b", Sb, Sb2, m, n)):
        K = np.sort(rng.choice(d, size=7, replace=False))
        X_K = O.factor_rows(G, Pa, Pb, K, side, mode)
        blk = O.factor_block(S[np.ix_(K, K)], X_K, 0.9482, 1e-9, den, mode)
        np.testing.assert_allclose(blk, S2[np.ix_(K, K)], rtol=1e-12, atol=1e-14)


def test_update_weights_rows_with_shape():
    rng = np.random.default_rng(13)
    W, U = rng.standard_normal((9, 14)), rng.standard_normal((9, 14))
    full = O.update_weights(W, U, 0.05, 0.09, 0.03)
    rows = O.update_weights(W[[2, 5]], U[[2, 5]], 0.05, 0.09, 0.03, shape=W.shape)
    np.testing.assert_array_equal(rows, full[[2, 5]])


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
@pytest.mark.parametrize("root", ["exact", "ns"])
def test_orthogonal_equivariance(mode, root):
    rng = np.random.default_rng(13)
    m, n = 7, 5
    Q1, Q2 = _orth(rng, m), _orth(rng, n)
    hp = O.Hyper(eps=1e-3)
    W0 = rng.standard_normal((m, n))
    s1 = O.init_state(W0, hp.eps)
    s2 = O.init_state(Q1 @ W0 @ Q2.T, hp.eps)
    for t in range(1, 4):
        G = rng.standard_normal((m, n))
        r1 = O.step(s1, G, hp, t, mode, root)
        r2 = O.step(s2, Q1 @ G @ Q2.T, hp, t, mode, root)
        np.testing.assert_allclose(r2.U, Q1 @ r1.U @ Q2.T, atol=1e-9 * np.abs(r1.U).max())
        np.testing.assert_allclose(r2.state.Sa, Q1 @ r1.state.Sa @ Q1.T, atol=1e-11)
        np.testing.assert_allclose(r2.state.Pb, Q2 @ r1.state.Pb @ Q2.T, atol=1e-9 * np.abs(r1.state.Pb).max())
        np.testing.assert_allclose(r2.state.W, Q1 @ r1.state.W @ Q2.T, atol=1e-11)
        s1, s2 = r1.state, r2.state


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
def test_transpose_identity(mode):
    """The step on G^T with the a/b state swapped yields the transposed
    whitened update and swapped factors."""
    rng = np.random.default_rng(14)
    m, n = 6, 4
    hp = O.Hyper(eps=1e-3)
    s1 = O.init_state(rng.standard_normal((m, n)), hp.eps)
    s2 = O.init_state(s1.W.T.copy(), hp.eps)
    for t in range(1, 4):
        G = rng.standard_normal((m, n))
        r1 = O.step(s1, G, hp, t, mode)
        r2 = O.step(s2, G.T, hp, t, mode)
        np.testing.assert_allclose(r2.U, r1.U.T, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(r2.state.Sa, r1.state.Sb, rtol=1e-11)
        np.testing.assert_allclose(r2.state.Pb, r1.state.Pa, rtol=1e-9)
        s1, s2 = r1.state, r2.state
        s2.W = s1.W.T.copy()  # W differs by c_shape asymmetry; keep it aligned


def test_zero_gradient_step_is_pure_decay():
    rng = np.random.default_rng(15)
    W = rng.standard_normal((8, 3))
    hp = O.Hyper()
    r = O.okls_step(O.init_state(W, hp.eps), np.zeros_like(W), hp, 1)
    assert np.all(r.U == 0.0)
    np.testing.assert_array_equal(r.state.W, (1.0 - hp.lr * hp.weight_decay) * W)


def test_adamc_decay_uses_lr_over_peak():
    W = np.ones((2, 2))
    U = np.zeros((2, 2))
    Wn = O.update_weights(W, U, lr=0.05, lr_peak=0.1, wd=0.2)
    np.testing.assert_allclose(Wn, (1 - 0.05 * 0.2 * 0.5) * W, rtol=1e-15)


def test_batched_equals_per_matrix():
    rng = np.random.default_rng(16)
    hp = O.Hyper(eps=1e-4)
    Ws = [rng.standard_normal((5, 3)) for _ in range(3)]
    Gs = [rng.standard_normal((5, 3)) for _ in range(3)]
    states = [O.init_state(w, hp.eps) for w in Ws]
    rb = O.step_batched(states, Gs, hp, 1)
    for i in range(3):
        ri = O.okls_step(O.init_state(Ws[i], hp.eps), Gs[i], hp, 1)
        np.testing.assert_array_equal(rb[i].state.W, ri.state.W)


# --------------------------------------------------------------------------
# Muon (R16): the un-accumulated Shampoo step through matrix products only.
# --------------------------------------------------------------------------
def test_muon_is_the_unaccumulated_shampoo_step_on_the_worked_example():
    """The Shampoo chapter: with one gradient and no accumulation the step
    L^{-1/4} G R^{-1/4} has singular values 1, 1, and Muon reaches that matrix
    with products alone.  A converged iteration (12 steps) equals the exact
    -1/4 step built from eigh roots; the Muon configuration (5 steps) keeps
    both singular values within its final half-width of 1."""
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    L, R = G @ G.T, G.T @ G
    Lq = O.inv_root_exact(L, 4)[0]
    # R is rank 2 (3 x 3): the -1/4 step acts on its range only
    lam, V = np.linalg.eigh(R)
    keep = lam > 1e-9 * lam.max()
    Rq = (V[:, keep] * lam[keep] ** -0.25) @ V[:, keep].T
    step_exact = Lq @ G @ Rq
    np.testing.assert_allclose(np.linalg.svd(step_exact, compute_uv=False), g["singular_values_preconditioned_one_accumulation"],
                               atol=g["printed_precision"])
    coeffs12, err12 = O.ns_coefficients(1e-2, 12)
    assert err12 < 1e-12
    np.testing.assert_allclose(O.ns_polar(G, coeffs12), step_exact, atol=1e-12)
    coeffs5, err5 = O.ns_coefficients(1e-2, 5)
    sv = np.linalg.svd(O.ns_polar(G, coeffs5), compute_uv=False)
    assert np.all(np.abs(sv - 1.0) <= err5 + 1e-12) and np.all(np.abs(sv - 1.0) < 0.05), sv


@pytest.mark.parametrize("shape", [(7, 5), (5, 7), (6, 6)])
def test_polar_iteration_converges_to_svd_polar_factor(shape):
    """Many steps reach U V^T from LAPACK's SVD (a different routine from the
    products the iteration uses), for both Gram orientations."""
    rng = np.random.default_rng(61)
    m, n = shape
    k = min(m, n)
    u, _ = np.linalg.qr(rng.standard_normal((m, k)))
    v, _ = np.linalg.qr(rng.standard_normal((n, k)))
    N = (u * np.logspace(0, -1.5, k)) @ v.T
    coeffs, err = O.ns_coefficients(1e-3, 14)
    assert err < 1e-10
    np.testing.assert_allclose(O.ns_polar(N, coeffs), u @ v.T, atol=1e-9)


def test_polar_five_steps_is_the_scalar_map_on_singular_values():
    """After 5 steps every singular value sigma has become p(sigma / c) with
    c = (sum sigma^4)^{1/4} and p the composed cubic steps; singular vectors
    are untouched (SVD route, not the products)."""
    rng = np.random.default_rng(62)
    m, n = 9, 13
    u, _ = np.linalg.qr(rng.standard_normal((m, m)))
    v, _ = np.linalg.qr(rng.standard_normal((n, m)))
    sig = np.exp(rng.uniform(-3, 0, m))
    N = (u * sig) @ v.T
    coeffs, _ = O.ns_coefficients(1e-2, 5)
    s = sig / np.sum(sig ** 4) ** 0.25
    for a, b in coeffs:
        s = s * (a + b * s * s)
    np.testing.assert_allclose(O.ns_polar(N, coeffs), (u * s) @ v.T, atol=1e-13)


def test_muon_step_is_scale_free_and_transposes():
    """Problem 14's point for the -1/4 step holds for Muon: G and 10 G give the
    same update; the transposed gradient gives the transposed update."""
    rng = np.random.default_rng(63)
    G = rng.standard_normal((6, 10))
    hp = O.muon_hyper()
    st = O.init_state(np.zeros((6, 10)), hp.eps)
    stT = O.init_state(np.zeros((10, 6)), hp.eps)
    r1 = O.muon_step(st, G, hp, 1)
    r10 = O.muon_step(st, 10.0 * G, hp, 1)
    rT = O.muon_step(stT, G.T, hp, 1)
    np.testing.assert_allclose(r10.U, r1.U, atol=1e-13)
    np.testing.assert_allclose(rT.U, r1.U.T, atol=1e-13)
    # t = 1: N = G (R5), W' = decay W - lr c_shape U from W = 0
    np.testing.assert_allclose(r1.N, G, atol=1e-15)
    np.testing.assert_allclose(r1.state.W, -hp.lr * O.c_shape(6, 10) * r1.U, atol=1e-15)
    # the factors and roots of the state are left as they were
    assert r1.state.Sa is st.Sa and r1.state.Pb is st.Pb


def test_muon_step_orthogonal_equivariance():
    rng = np.random.default_rng(64)
    G = rng.standard_normal((5, 8))
    Qa, Qb = _orth(rng, 5), _orth(rng, 8)
    hp = O.muon_hyper()
    st = O.init_state(rng.standard_normal((5, 8)), hp.eps)
    stQ = O.init_state(Qa @ st.W @ Qb.T, hp.eps)
    r = O.muon_step(st, G, hp, 1)
    rQ = O.muon_step(stQ, Qa @ G @ Qb.T, hp, 1)
    np.testing.assert_allclose(rQ.U, Qa @ r.U @ Qb.T, atol=1e-12)


# ---------------------------------------------------------------------------
# Readings kept as configuration switches (R1 convex eps, R6 decay order,
# R7 plain update).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("convex", [False, True])
def test_eps_placement_zero_gradient_closed_form(convex):
    """Zero gradients from S_0 = eps I: X = 0, so each update only rescales S
    and adds the eps term.  Literal R1 (+ eps I): S_t = (beta2^t + (1 - beta2^t)
    / (1 - beta2)) eps I, a geometric series tending to eps / (1 - beta2).
    Convex (+ (1 - beta2) eps I): eps I is a fixed point, S_t = eps I."""
    m, n, eps, beta2 = 5, 3, 1e-9, 0.9482
    hp = O.Hyper(eps=eps, beta2=beta2, eps_convex=convex)
    st = O.init_state(np.zeros((m, n)), eps)
    for t in range(1, 41):
        st = O.okls_step(st, np.zeros((m, n)), hp, t).state
        want = eps if convex else eps * (beta2 ** t + (1.0 - beta2 ** t) / (1.0 - beta2))
        np.testing.assert_allclose(st.Sa, want * np.eye(m), rtol=1e-12, atol=0)
        np.testing.assert_allclose(st.Sb, want * np.eye(n), rtol=1e-12, atol=0)
    blk = O.factor_block(eps * np.eye(2), np.zeros((2, 4)), beta2, eps, 4, "okls", eps_convex=convex)
    np.testing.assert_allclose(blk, (eps if convex else (beta2 + 1.0) * eps) * np.eye(2), rtol=1e-12)


def test_decay_after_scales_the_whole_step():
    """R6's two orders differ only in what the decay multiplies.  With a zero
    update both give decay * W; from W = 0 the decay-after step is exactly
    decay times the decay-free step (the update term is decayed too), while
    the decay-before step equals the decay-free one."""
    rng = np.random.default_rng(61)
    W, U = rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    lr, peak, wd = 0.05, 0.1, 0.2
    decay = 1.0 - lr * wd * lr / peak
    for after in (False, True):
        np.testing.assert_allclose(O.update_weights(W, 0 * U, lr, peak, wd, decay_after=after), decay * W, rtol=1e-15)
    free = O.update_weights(0 * W, U, lr, peak, 0.0)
    np.testing.assert_allclose(O.update_weights(0 * W, U, lr, peak, wd, decay_after=True), decay * free, rtol=1e-14)
    np.testing.assert_allclose(O.update_weights(0 * W, U, lr, peak, wd, decay_after=False), free, rtol=1e-15)


def test_plain_shampoo_update_reproduces_the_worked_example_in_the_weights():
    """R7's alternative, the original Shampoo step: no momentum (beta1 = 0,
    no variance correction), no decay, no c_shape.  With lr = 1, W_0 = 0 and
    the worked example's G repeated, the step W_{t-1} - W_t is
    L^{-1/4} G R^{-1/4} itself, so its singular values are the page's: 1, 1
    after one accumulation, 0.5 after four and 0.1 after a hundred."""
    g = _gold("shampoo_worked_example.json")
    G = np.array(g["G"], dtype=np.float64)
    hp = O.Hyper(lr=1.0, beta1=0.0, nesterov_var_corr=False, weight_decay=0.0, shape_scale=False, eps=1e-12)
    st = O.init_state(np.zeros_like(G), hp.eps)
    want = {1: g["singular_values_preconditioned_one_accumulation"],
            4: g["singular_values_after_4_identical_accumulations"],
            100: g["singular_values_after_100_identical_accumulations"]}
    for t in range(1, 101):
        W_prev = st.W
        st = O.shampoo_step(st, G, hp, t).state
        if t in want:
            sv = np.linalg.svd(W_prev - st.W, compute_uv=False)
            np.testing.assert_allclose(sv, want[t], atol=g["printed_precision"])
            np.testing.assert_allclose(sv, [t ** -0.5] * 2, atol=1e-6)
    # the default (muP) step is the same update scaled by c_shape(2, 3)
    st0 = O.init_state(np.zeros_like(G), hp.eps)
    plain = O.shampoo_step(st0, G, hp, 1).state.W
    scaled = O.shampoo_step(st0, G, O.Hyper(lr=1.0, beta1=0.0, nesterov_var_corr=False, weight_decay=0.0,
                                           eps=1e-12), 1).state.W
    np.testing.assert_allclose(scaled, O.c_shape(2, 3) * plain, rtol=1e-12)


def test_classical_coefficients_converge_to_the_exact_root():
    """R4's classical alternative, T = (3 I - Z Y) / 2 at every step: sigma = 1
    is its fixed point, and on a well-conditioned factor (kappa 10, spectrum
    in (0, 1] after the Frobenius scaling) the coupled iteration converges
    quadratically to the exact eigh inverse square root."""
    coeffs, err = O.ns_coefficients(1e-3, 25, classical=True)
    assert err is None and coeffs == [(1.5, -0.5)] * 25
    assert 1.0 * (1.5 - 0.5 * 1.0) == 1.0
    rng = np.random.default_rng(71)
    Q, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    S = (Q * np.linspace(0.1, 1.0, 12)) @ Q.T
    P, _ = O.ns_inv_sqrt(S, coeffs, 0.0)
    exact, _ = O.inv_root_exact(S, 2)
    assert O.rel_frob(P, exact) < 1e-12
    # and the per-eigenvalue closed form follows the same table
    np.testing.assert_allclose(O.ns_eigen_closed_form(S, coeffs, 2, 0.0), P, rtol=1e-10, atol=1e-12)
    hp = O.Hyper(ns_classical=True, ns_steps=7)
    assert hp.coeffs() == [(1.5, -0.5)] * 7


def test_ns_residual_hand_computed():
    """Classical Newton-Schulz (a, b) = (3/2, -1/2) on S = 3 I of side 4:
    c = ||S||_F = 6, Y_0 = I / 2, so Z_0 Y_0 = I / 2 and the residual with
    K = 1 is ||-I / 2||_F = 1.  One step gives sigma^2 = (1/2)(3/2 - 1/4)^2 =
    25 / 32, so with K = 2 the residual (of Z_1 Y_1) is 2 (1 - 25/32) = 7/16."""
    S = 3.0 * np.eye(4)
    assert O.ns_residual(S, [(1.5, -0.5)]) == pytest.approx(1.0, abs=1e-15)
    assert O.ns_residual(S, [(1.5, -0.5)] * 2) == pytest.approx(7.0 / 16.0, abs=1e-15)


@pytest.mark.parametrize("nu", [0.0, 5e-3])
def test_ns_residual_matches_the_eigenvalue_recurrence(nu):
    """The matrix iteration's ||Z_{K-1} Y_{K-1} - I||_F equals the residual of
    the scalar recurrence over S's eigenvalues (LAPACK eigh), and falls as
    classical steps are added on a well-conditioned factor (there 1 - sigma^2
    shrinks at every step in every direction)."""
    rng = np.random.default_rng(41)
    coeffs, _ = O.ns_coefficients(1e-3, 10)
    for d, kappa in ((30, 1e2), (64, 1e4)):
        S = _spd(rng, d, kappa) * 0.7
        r = O.ns_residual(S, coeffs, nu)
        lam = np.linalg.eigvalsh(S)
        assert r == pytest.approx(O.ns_residual_spectral(lam, coeffs, nu), rel=1e-9, abs=1e-12)
    S = _spd(rng, 40, 10.0)
    seq = [O.ns_residual(S, [(1.5, -0.5)] * k, nu) for k in range(1, 11)]
    assert all(b < a for a, b in zip(seq, seq[1:])) and seq[-1] < 1e-12
