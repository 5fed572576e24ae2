"""CPU checks of the seeded input generators: shapes, seeds, distributions
and the known-spectrum factor construction used by the full-size checks."""
import math

import numpy as np
import pytest

from kronecker_factored_second_amd import workloads as WL


def test_random_orthogonal_is_orthogonal_and_dense():
    Q = WL.RandomOrthogonal(np.random.default_rng(0), 257)
    M = Q.apply(np.eye(257))
    np.testing.assert_allclose(M.T @ M, np.eye(257), atol=1e-13)
    np.testing.assert_allclose(Q.apply_t(np.eye(257)), M.T, atol=1e-14)
    np.testing.assert_allclose(Q.rows([0, 100, 256]), M[[0, 100, 256]], atol=1e-14)
    X = np.random.default_rng(1).standard_normal((4, 257))
    np.testing.assert_allclose(Q.apply(X, axis=1), X @ M.T, atol=1e-13)
    # no eigenvector concentrates on a few coordinates
    assert np.max(np.abs(M)) < 0.5


def test_symmetric_from_spectrum_dense_and_rows():
    rng = np.random.default_rng(2)
    Q = WL.RandomOrthogonal(rng, 96)
    lam = np.exp(rng.uniform(-6, 0, 96))
    M = Q.apply(np.eye(96))
    S = WL.symmetric_from_spectrum(Q, lam)
    np.testing.assert_allclose(S, (M * lam) @ M.T, atol=1e-15)
    assert np.array_equal(S, S.T)
    np.testing.assert_allclose(np.sort(np.linalg.eigvalsh(S)), np.sort(lam), rtol=1e-9)
    np.testing.assert_allclose(WL.symmetric_from_spectrum(Q, lam, rows=[3, 50]), S[[3, 50]], atol=1e-15)


def test_spectral_factor_endpoints_and_seed():
    Q, lam = WL.spectral_factor("c3", 1, 0, 0, 300, 1e4, 2e-5)
    assert lam.max() == 2e-5 and math.isclose(lam.min(), 2e-9)
    Q2, lam2 = WL.spectral_factor("c3", 1, 0, 0, 300, 1e4, 2e-5)
    assert np.array_equal(lam, lam2)
    np.testing.assert_array_equal(Q.apply(np.eye(300)[:, 7]), Q2.apply(np.eye(300)[:, 7]))


def test_illcond_gradient_spectrum():
    """A Z B with log-spaced singular values of A and B on [1e-3, 1]."""
    w = WL.Workload("c5", [(192, 128, 1)], "okls", "illcond", "f32", 1, (1,))
    WL.reset_caches()
    G = WL.gradient(w, 0, 0, 1).astype(np.float64)
    WL.reset_caches()
    assert np.array_equal(G, WL.gradient(w, 0, 0, 1))
    sv = np.linalg.svd(G, compute_uv=False)
    assert 1e3 < sv.max() / sv.min() < 1e7


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_workload_shapes(name):
    w = WL.workload(name)
    d, f = {"c2": (1024, 2816), "c3": (2048, 5632), "c4": (4096, 11008), "c5": (5120, 13824)}[name]
    layers = {"c2": 1, "c3": 24, "c4": 32, "c5": 1}[name]
    assert w.groups == [(d, d, 4 * layers), (f, d, 2 * layers), (d, f, layers)]
    assert w.n_matrices == 7 * layers
