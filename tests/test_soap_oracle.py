"""Pins of the fp64 eigenbasis-Adam (SOAP) oracle against what the pages and
the mathematics fix: the Shampoo chapter's worked example, closed forms of
Adam on a constant gradient, the 2 x 2 eigenvector angle, the SVD polar
factor (the refreshed step with no averaging), orthogonal equivariance and
unrolled sums of the moments over changing bases.  No GPU is needed.
"""
import json
import math
import os

import numpy as np
import scipy.linalg

from oracle import soap_oracle as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _orth(rng, d):
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    return Q * np.sign(np.diag(R))


def _random_state(rng, m, n):
    """A state with SPD factors of distinct eigenvalues and bases that are
    their eigenvectors (as after a refresh), non-zero moments."""
    st = S.init_state(rng.standard_normal((m, n)))
    QL, QR = _orth(rng, m), _orth(rng, n)
    st.L = (QL * np.linspace(1.0, 2.0, m)) @ QL.T
    st.R = (QR * np.linspace(1.0, 3.0, n)) @ QR.T
    st.QL, st.QR = QL, QR
    st.M = rng.standard_normal((m, n))
    st.V = rng.random((m, n)) + 0.1
    return st


def test_adam_constant_gradient_bias_corrected():
    """A constant gradient makes the corrected moments exactly G' and G'^2:
    N' = G'/(|G'| + eps) at every step (S1), here in the initial basis Q = I."""
    rng = np.random.default_rng(0)
    G = rng.standard_normal((4, 6))
    hp = S.SoapHyper(freq=1000, eps=1e-3, weight_decay=0.0)
    st = S.init_state(np.zeros((4, 6)))
    for t in range(1, 7):
        r = S.soap_step(st, G, hp, t)
        np.testing.assert_allclose(r.N_rot, G / (np.abs(G) + hp.eps), rtol=1e-12, atol=0)
        np.testing.assert_allclose(r.N, r.N_rot, rtol=0, atol=0)     # Q = I before the first refresh (S3)
        st = r.state


def test_adam_constant_gradient_uncorrected():
    """Without the corrections the EMAs of a constant are geometric sums:
    M_t = (1 - b1^t) G, V_t = (1 - b2^t) G^2."""
    rng = np.random.default_rng(1)
    G = rng.standard_normal((3, 5))
    hp = S.SoapHyper(freq=1000, eps=1e-3, weight_decay=0.0, bias_correction=False, beta1=0.8, beta2=0.6)
    st = S.init_state(np.zeros((3, 5)))
    for t in range(1, 6):
        r = S.soap_step(st, G, hp, t)
        want = (1 - 0.8 ** t) * G / (math.sqrt(1 - 0.6 ** t) * np.abs(G) + hp.eps)
        np.testing.assert_allclose(r.N_rot, want, rtol=1e-12)
        st = r.state


def test_weight_update_form():
    """S5: a zero gradient from zero moments leaves N = 0 and W' = (1 - lr wd) W."""
    rng = np.random.default_rng(2)
    st = S.init_state(rng.standard_normal((3, 4)))
    hp = S.SoapHyper(lr=0.01, weight_decay=0.5, freq=1000)
    r = S.soap_step(st, np.zeros((3, 4)), hp, 1)
    np.testing.assert_array_equal(r.N, np.zeros((3, 4)))
    np.testing.assert_allclose(r.state.W, (1 - 0.005) * st.W, rtol=1e-15)


def test_factor_update_worked_example():
    """The Shampoo chapter's 2 x 3 worked example: L = G G^T = [[10, 3], [3, 5]]
    (one update with beta = 0)."""
    with open(os.path.join(GOLD, "shampoo_worked_example.json")) as f:
        g = json.load(f)
    G = np.array(g["G"], dtype=np.float64)
    L, R = S.factor_update(np.zeros((2, 2)), np.zeros((3, 3)), G, 0.0)
    np.testing.assert_allclose(L, g["L_equals_G_GT"], atol=1e-12)
    np.testing.assert_allclose(np.sort(np.linalg.eigvalsh(R))[1:], np.sort(np.linalg.eigvalsh(L)), atol=1e-12)


def test_factor_update_unrolled():
    rng = np.random.default_rng(3)
    Gs = [rng.standard_normal((4, 3)) for _ in range(5)]
    b = 0.7
    L, R = np.zeros((4, 4)), np.zeros((3, 3))
    for G in Gs:
        L, R = S.factor_update(L, R, G, b)
    Lw = np.zeros((4, 4))
    Rw = np.zeros((3, 3))
    for s, G in enumerate(Gs):
        w = (1 - b) * b ** (len(Gs) - 1 - s)
        for j in range(G.shape[1]):       # G G^T as a sum of column outer products
            Lw += w * np.outer(G[:, j], G[:, j])
        for i in range(G.shape[0]):       # G^T G as a sum of row outer products
            Rw += w * np.outer(G[i], G[i])
    np.testing.assert_allclose(L, Lw, rtol=1e-12)
    np.testing.assert_allclose(R, Rw, rtol=1e-12)


def test_eigenvectors_follow_the_warm_start():
    """S2: a diagonal matrix with distinct entries keeps an identity or a
    signed-permutation warm start exactly."""
    A = np.diag([3.0, 1.0, 4.0, 1.5, 9.0])
    np.testing.assert_array_equal(S.eigenvectors(A, np.eye(5)), np.eye(5))
    P = np.eye(5)[:, [2, 0, 4, 1, 3]] * np.array([1, -1, -1, 1, 1])
    np.testing.assert_array_equal(S.eigenvectors(A, P), P)


def test_eigenvectors_2x2_angle():
    """The symmetric 2 x 2 [[a, b], [b, c]] has its larger eigenvalue's vector
    at angle theta = atan2(2b, a - c) / 2 (the Jacobi rotation angle)."""
    for a, b, c in [(3.0, 0.4, 1.0), (2.0, -0.7, 1.5), (1.0, 0.2, 5.0)]:
        th = 0.5 * math.atan2(2 * b, a - c)
        big = np.array([math.cos(th), math.sin(th)])
        Q = S.eigenvectors(np.array([[a, b], [b, c]]), np.eye(2))
        j = int(np.argmax(np.abs(Q.T @ big)))
        assert abs(abs(Q[:, j] @ big) - 1.0) < 1e-14
        lam_big = 0.5 * (a + c) + math.hypot(0.5 * (a - c), b)
        np.testing.assert_allclose(Q[:, j] @ np.array([[a, b], [b, c]]) @ Q[:, j], lam_big, rtol=1e-14)
        assert np.all(np.diag(Q) > 0)      # signs follow the identity warm start


def test_eigenvectors_random_spd_invariants():
    rng = np.random.default_rng(4)
    d = 12
    E = _orth(rng, d)
    A = (E * np.linspace(0.5, 6.0, d)) @ E.T
    # warm start: the eigenbasis rotated slightly, columns shuffled, signs flipped
    perm = rng.permutation(d)
    K = 1e-2 * rng.standard_normal((d, d))
    warm = E[:, perm] * np.where(rng.random(d) < 0.5, -1.0, 1.0)
    warm = warm @ scipy.linalg.expm(K - K.T)
    Q = S.eigenvectors(A, warm)
    assert S.offdiag_residual(Q, A) < 1e-14
    assert S.orthogonality(Q) < 1e-14
    # each column stays with the warm-start column it came from
    assert np.all(np.sum(Q * warm, axis=0) > 0.99)


def test_refreshed_step_is_the_polar_factor():
    """With no averaging (beta1 = beta2 = shampoo beta = 0) and bases refreshed
    from G G^T and G^T G, the next step on the same G rotates G to its signed
    singular values; the Adam ratio sets each to +-1 and the step back is the
    polar factor U V^T of G (scipy's polar decomposition).  eps sits between
    the rounding residue of the zero entries (~1e-15) and the singular values."""
    rng = np.random.default_rng(5)
    for m, n in [(5, 8), (7, 4), (6, 6)]:
        G = rng.standard_normal((m, n))
        hp = S.SoapHyper(beta1=0.0, beta2=0.0, shampoo_beta=0.0, freq=1, weight_decay=0.0, eps=1e-7)
        st = S.init_state(np.zeros((m, n)))
        st = S.soap_step(st, G, hp, 1).state
        r = S.soap_step(st, G, hp, 2)
        if m <= n:
            u, _ = scipy.linalg.polar(G, side="left")      # G = p u, u has orthonormal rows
        else:
            u, _ = scipy.linalg.polar(G)                   # G = u p, u has orthonormal columns
        np.testing.assert_allclose(r.N, u, atol=1e-6)


def test_step_equivariance():
    """Rotating the problem (W, M, G by O_m . O_n^T; L, Q_L by O_m; R, Q_R by
    O_n) rotates every output; V, the eigenbasis coordinates, is unchanged.
    Two steps, the second refreshing the bases."""
    rng = np.random.default_rng(6)
    m, n = 5, 7
    Om, On = _orth(rng, m), _orth(rng, n)
    st = _random_state(rng, m, n)
    sr = S.SoapState(W=Om @ st.W @ On.T, M=Om @ st.M @ On.T, V=st.V.copy(), L=Om @ st.L @ Om.T,
                     R=On @ st.R @ On.T, QL=Om @ st.QL, QR=On @ st.QR)
    hp = S.SoapHyper(freq=2, lr=0.05, eps=1e-6)
    for t in (1, 2):
        G = rng.standard_normal((m, n))
        a = S.soap_step(st, G, hp, t)
        b = S.soap_step(sr, Om @ G @ On.T, hp, t)
        np.testing.assert_allclose(b.state.W, Om @ a.state.W @ On.T, atol=1e-12)
        np.testing.assert_allclose(b.state.M, Om @ a.state.M @ On.T, atol=1e-12)
        np.testing.assert_allclose(b.state.V, a.state.V, atol=1e-12)
        np.testing.assert_allclose(b.state.L, Om @ a.state.L @ Om.T, atol=1e-12)
        np.testing.assert_allclose(b.state.QL, Om @ a.state.QL, atol=1e-10)
        np.testing.assert_allclose(b.state.QR, On @ a.state.QR, atol=1e-10)
        np.testing.assert_allclose(b.N_rot, a.N_rot, atol=1e-12)
        st, sr = a.state, b.state
    assert a.refreshed


def test_moment_bases_unrolled():
    """S4 over a refresh: Algorithm 4's M' is the current basis applied to the
    parameter-space EMA of all gradients; the eigenbasis variant sums each
    gradient rotated in the basis of its own step.  V sums the squared
    rotated gradients of each step's basis in both."""
    rng = np.random.default_rng(7)
    m, n, T = 4, 6, 5
    Gs = [rng.standard_normal((m, n)) for _ in range(T)]
    for moments in ("param", "eigen"):
        hp = S.SoapHyper(freq=2, beta1=0.7, beta2=0.6, shampoo_beta=0.5, moments=moments)
        st = S.init_state(np.zeros((m, n)))
        bases = []
        for t, G in enumerate(Gs, start=1):
            bases.append((st.QL, st.QR))
            r = S.soap_step(st, G, hp, t)
            st = r.state
        w1 = [(1 - 0.7) * 0.7 ** (T - 1 - s) for s in range(T)]
        w2 = [(1 - 0.6) * 0.6 ** (T - 1 - s) for s in range(T)]
        QL, QR = bases[-1]
        if moments == "param":
            want = QL.T @ sum(w * G for w, G in zip(w1, Gs)) @ QR
        else:
            want = sum(w * (ql.T @ G @ qr) for w, G, (ql, qr) in zip(w1, Gs, bases))
        np.testing.assert_allclose(r.M_rot, want, atol=1e-12)
        Vw = sum(w * (ql.T @ G @ qr) ** 2 for w, G, (ql, qr) in zip(w2, Gs, bases))
        np.testing.assert_allclose(st.V, Vw, atol=1e-12)
        # refreshes after steps 2 and 4 (t % f == 0) only
        assert np.array_equal(bases[1][0], bases[0][0]) and np.array_equal(bases[3][0], bases[2][0])
        assert not np.allclose(bases[2][0], bases[1][0]) and not np.allclose(bases[4][0], bases[3][0])
