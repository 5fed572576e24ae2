"""Plain fp64 CPU oracle of the Nystrom low-rank factor step (Clean's
low-rank Kronecker factors with the Nystrom preconditioner).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers
with the HIP library; the two meet only at seeded inputs (the Gaussian
sketch matrices are inputs of both).

Passages followed ("Clean: Second-order LLM Training at Linear Memory Cost
via Nystrom Sketching"; short name [CLEAN]):
  [NYS]   section 2.2: the randomized Nystrom approximation (eq. 4) and the
          Nystrom preconditioner P = (lambda_r + mu)^-1 U (Lambda + mu I) U^T
          + (I - U U^T) (eq. 5).
  [LOWR]  section 3, "Smoothed covariances" and "Low-rank covariance
          factors": L_t = beta2 L_{t-1} + (1 - beta2) G G^T (eq. 6), stored
          only as U Lambda U^T (eq. 7), the sketch of eq. (8) through the
          stored factors, refreshed every T steps, Algorithm 1's first lines
          (a refresh when (t - 1) mod T == 0, before the step uses them).
  [BLOCK] section 3, "Block-wise low-rank preconditioning": G_pre =
          L^-1/2 G R^-1/2 with P^-1/2 = c U D U^T + P_perp (eq. 9-10),
          D = (Lambda + mu I)^-1/2, c = (lambda_r + mu)^1/2.
  [ALG2]  Appendix A, Algorithm 2 (randomized Nystrom approximation): thin QR
          of the test matrix, shift nu = eps(||Y||_2), Cholesky of the
          symmetrised B, triangular solve, thin SVD, eigenvalues max(0,
          Sigma^2 - nu).
  [ALG3]  Appendix A, Algorithm 3 (warm start [U_prev, Psi], q passes of
          subspace iteration with re-orthonormalisation, the final sketch,
          the steps of Algorithm 2, the oversampling discarded, signs aligned
          with U_prev).

Readings where the pages leave a step open (listed with the design notes as
N1..N9):
  N1  eps(x) is the spacing of IEEE single precision at x, 2^(floor(log2 x)
      - 23): the shift is meant at the working precision's rounding level,
      and the library works in fp32.
  N2  Algorithm 3's QR after the if/else applies to both branches (the warm
      start [U_prev, Psi] is orthonormalised too).
  N3  mu (eq. 5, 9) is the library's eps, the regularisation the other modes
      add to their factors.
  N4  The preconditioned matrix is the library's momentum N (the Nesterov
      reading of the OKLS mode; beta1 = 0 without variance correction gives
      G, eq. 9 as printed); the update is the OKLS one, W <- decay W - lr
      c_shape U with U = P_L^-1/2 N P_R^-1/2.  Clean's four-block Adam (its
      Table 1, eq. 12-16) is not part of this step.
  N5  The Gaussian matrices of a refresh are inputs: Psi_L (m x (r + p)) and
      Psi_R (n x (r + p)); a warm start takes their first p columns, a cold
      start (no previous factors) all r + p.
  N6  Before the first refresh the factors are empty (Lambda = 0, no U):
      the t = 1 refresh is a cold start on A = (1 - beta2) G G^T.
  N7  A side d smaller than r + p sketches with k = d columns and keeps
      min(r, d) of them.
  N8  A sketch Y = 0 (a zero factor) gives Lambda = 0 and U = the first
      columns of the orthonormalised test matrix (nothing to factor).
  N9  With r above the factor's rank the tail eigenvalues are zero here
      (fp64: ~1e-17 of ||A||) but sit at the sketch's rounding level in any
      fp32 computation (~nu), and c = (lambda_r + mu)^1/2 follows that
      rounding unless mu is far above nu: P^-1/2 is then defined by the
      arithmetic, not by the method.  Comparisons keep r at or below the
      factors' rank.

Parity status (what pins each function in the CPU test-suite):
  nystrom (Alg. 2/3) ... an exactly rank-r PSD matrix is reproduced to
                         rounding; the warm start equals the cold start after
                         enough passes on a matrix with a spectral gap; q = 0
                         cold start is Algorithm 2; eigenvalues within the
                         shift of the exact ones for a rank <= r matrix
  inv_sqrt_precond ..... identity on the orthogonal complement, c D on U;
                         with r = d it is sqrt(lambda_r + mu) (A + mu I)^-1/2,
                         the exact-root Shampoo factor (LAPACK eigh of A)
  precondition ......... equals (P_L^-1/2) N (P_R^-1/2) formed densely; with
                         full rank it is the exact-root Shampoo whitening
  nys_step ............. refresh schedule and sign alignment; W update form
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

from oracle.okls_oracle import c_shape, momentum


@dataclass
class NysHyper:
    lr: float = 1e-2
    beta1: float = 0.9684            # momentum as the OKLS mode ([OKLS README] defaults)
    beta2: float = 0.95              # [LOWR] eq. 6 EMA coefficient ([CLEAN] Table 6's 0.95)
    eps: float = 1e-9                # mu, N3
    weight_decay: float = 0.0303
    lr_peak: float | None = None
    nesterov_var_corr: bool = True
    shape_scale: bool = True
    rank: int = 32                   # r
    oversample: int = 8              # p
    passes: int = 1                  # q
    period: int = 10                 # T ([CLEAN] Table 6 / its Appendix E: T = 10)

    def peak(self) -> float:
        return self.lr if self.lr_peak is None else self.lr_peak

    def refresh(self, t: int) -> bool:
        """[LOWR] Algorithm 1: refresh when (t - 1) mod T == 0."""
        return (t - 1) % max(self.period, 1) == 0


def eps32(x: float) -> float:
    """N1: spacing of IEEE single precision at x > 0."""
    if x <= 0.0:
        return 0.0
    return math.ldexp(1.0, math.floor(math.log2(x)) - 23)


def thin_qr(X):
    """Thin QR (LAPACK Householder via numpy), Q with X = Q R."""
    q, _ = np.linalg.qr(X, mode="reduced")
    return q


def sketch_size(d: int, r: int, p: int):
    """N7: (k, kept) columns for a side d."""
    k = min(r + p, d)
    return k, min(r, k)


def nystrom(apply_A, m: int, r: int, p: int, q: int, U_prev, Psi):
    """[ALG3] with [ALG2]'s final steps.  apply_A(X) = A X for the PSD A;
    Psi is m x (r + p) Gaussian (N5).  Returns (U, Lambda, nu)."""
    k, r = sketch_size(m, r, p)
    if U_prev is not None:
        Om = np.concatenate([U_prev, Psi[:, :k - U_prev.shape[1]]], axis=1)
    else:
        Om = Psi[:, :k]
    Om = thin_qr(Om)                                  # N2
    for _ in range(q):
        Y = apply_A(Om)
        Om = thin_qr(Y)
    Y = apply_A(Om)
    if not np.any(Y):                                 # N8
        return Om[:, :r], np.zeros(r), 0.0
    nu = eps32(float(np.linalg.norm(Y, 2)))
    Ynu = Y + nu * Om
    B = Om.T @ Ynu
    C = np.linalg.cholesky(0.5 * (B + B.T)).T        # upper, C^T C = sym(B)
    F = np.linalg.solve(C.T, Ynu.T).T                 # Y_nu C^-1 (triangular solve)
    U, S, _ = np.linalg.svd(F, full_matrices=False)
    lam = np.maximum(0.0, S ** 2 - nu)
    U, lam = U[:, :r], lam[:r]
    if U_prev is not None:
        s = np.sign(np.sum(U * U_prev[:, :r], axis=0))
        s[s == 0] = 1.0
        U = U * s
    return U, lam, nu


def nystrom_alg2(A, r: int, Om):
    """[ALG2] as printed (test matrix given), for the pin that Algorithm 3
    with no warm start and q = 0 is Algorithm 2."""
    Om = thin_qr(Om)
    Y = A @ Om
    nu = eps32(float(np.linalg.norm(Y, 2)))
    Ynu = Y + nu * Om
    B = Om.T @ Ynu
    C = np.linalg.cholesky(0.5 * (B + B.T)).T
    F = np.linalg.solve(C.T, Ynu.T).T
    U, S, _ = np.linalg.svd(F, full_matrices=False)
    return U[:, :r], np.maximum(0.0, S ** 2 - nu)[:r]


def inv_sqrt_precond(U, lam, mu: float, d: int):
    """[NYS] eq. 5 / [BLOCK] eq. 9: P^-1/2 = c U D U^T + (I - U U^T), dense d x d."""
    c = math.sqrt(lam[-1] + mu)
    D = 1.0 / np.sqrt(lam + mu)
    return c * (U * D) @ U.T + (np.eye(d) - U @ U.T)


def precondition(UL, lamL, UR, lamR, N, mu: float):
    """[BLOCK] eq. 10: P_L^-1/2 N P_R^-1/2 (formed densely here)."""
    m, n = N.shape
    return inv_sqrt_precond(UL, lamL, mu, m) @ N @ inv_sqrt_precond(UR, lamR, mu, n)


@dataclass
class NysState:
    W: np.ndarray
    M: np.ndarray
    UL: np.ndarray | None = None     # m x r (None before the first refresh, N6)
    lamL: np.ndarray | None = None
    UR: np.ndarray | None = None
    lamR: np.ndarray | None = None


def init_state(W) -> NysState:
    W = np.array(W, dtype=np.float64)
    return NysState(W=W, M=np.zeros_like(W))


@dataclass
class NysResult:
    state: NysState
    N: np.ndarray
    U: np.ndarray
    nu: tuple = (0.0, 0.0)
    extra: dict = field(default_factory=dict)


def nys_step(st: NysState, G, hp: NysHyper, t: int, PsiL=None, PsiR=None) -> NysResult:
    """One step for one matrix: the factor refresh on schedule ([LOWR], [ALG3]),
    the momentum (N4), the preconditioned U = P_L^-1/2 N P_R^-1/2 ([BLOCK]),
    the OKLS update W <- decay W - lr c_shape U."""
    G = np.asarray(G, dtype=np.float64)
    m, n = G.shape
    r, p, q, b2 = hp.rank, hp.oversample, hp.passes, hp.beta2
    UL, lamL, UR, lamR = st.UL, st.lamL, st.UR, st.lamR
    nu = (0.0, 0.0)
    if hp.refresh(t):
        def left(X, U=UL, lam=lamL):      # (b2 U Lambda U^T + (1 - b2) G G^T) X, eq. 8
            out = (1.0 - b2) * (G @ (G.T @ X))
            if U is not None:
                out = out + b2 * (U * lam) @ (U.T @ X)
            return out

        def right(X, U=UR, lam=lamR):
            out = (1.0 - b2) * (G.T @ (G @ X))
            if U is not None:
                out = out + b2 * (U * lam) @ (U.T @ X)
            return out

        UL, lamL, nuL = nystrom(left, m, r, p, q, UL, PsiL)
        UR, lamR, nuR = nystrom(right, n, r, p, q, UR, PsiR)
        nu = (nuL, nuR)
    M, N = momentum(st.M, G, hp.beta1, t, hp.nesterov_var_corr)     # N4: the OKLS mode's momentum
    U = precondition(UL, lamL, UR, lamR, N, hp.eps)
    decay = 1.0 - hp.lr * hp.weight_decay * (hp.lr / hp.peak())
    c = c_shape(m, n) if hp.shape_scale else 1.0
    W = decay * st.W - hp.lr * c * U
    return NysResult(NysState(W, M, UL, lamL, UR, lamR), N, U, nu)
