"""Plain fp64 CPU oracle of the eigenbasis-Adam step (SOAP; KPOP's Adam in
the Kronecker-factored eigenbasis).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers
with the HIP library; the two meet only at seeded inputs.

Passages followed (short names as in okls_oracle):

  [CLEAN-C]  "Clean: Second-order LLM Training at Linear Memory Cost via
             Nystrom Sketching", Appendix C, Algorithm 4 (SOAP): the gradient
             and the first moment rotated into the factors' eigenbasis, Adam's
             second moment kept there, the step rotated back, the factors
             updated after the step and their eigenvectors refreshed every f
             steps, Eigenvectors(L, Q_L) warm-started from the current basis.
  [CLEAN-T]  the same paper, Appendix F, Tables 4 and 6: SOAP's (beta1, beta2)
             = (0.95, 0.95), Shampoo beta 0.95, preconditioning frequency 10,
             learning rate 2.8e-3, Adam eps 1e-8, decoupled weight decay 0.1.
  [KPOP]     "KPOP Optimiser Explained", sections "Transforming the Gradient"
             (Adam with bias correction on the rotated gradient, step
             Q_R dW' Q_C^T) and "Updating Kronecker Factors During Training"
             (EMA factors, eigendecomposition of the EMA estimates).

Readings where the pages leave a step open (the design notes list them as
S1..S5):
  S1  Algorithm 4's line computing N' is garbled in the page's text; the
      reading is Adam's bias-corrected ratio as [KPOP] writes it,
      N' = (M'/(1 - beta1^t)) / (sqrt(V/(1 - beta2^t)) + eps).  Switch:
      bias_correction=False drops both corrections.
  S2  Eigenvectors(L, Q_L) returns an orthonormal eigenbasis of L whose
      columns follow the warm start: column j is the eigenvector that best
      matches column j of Q_L (largest squared overlap, one-to-one), with the
      sign that makes their inner product non-negative.  Where eigenvalues
      repeat the basis of their eigenspace is not unique; comparisons of a
      computed basis therefore use invariants (orthogonality, the residual of
      Q^T L Q off its diagonal) and alignment only for separated eigenvalues.
  S3  Initial state: L = R = 0, Q_L = Q_R = I, M = V = 0; so the steps before
      the first refresh (t < f) are Adam in the parameter basis.
  S4  Algorithm 4 keeps M in the parameter space and rotates it each step;
      [KPOP] keeps m in the eigenbasis (m' <- beta1 m' + (1 - beta1) G').
      Switch moments="eigen" selects the latter.
  S5  Weight decay: decoupled, W <- (1 - lr wd) W - lr N ([CLEAN-T] Table 4);
      wd = 0 is Algorithm 4's W <- W - lr N.

Parity status (what pins each function in the CPU test-suite):
  adam_direction ........ constant gradient: N' = G'/(|G'| + eps) at every t
                          (bias correction exact); no correction: the closed
                          form of the uncorrected EMAs of a constant
  eigenvectors .......... diagonal input and identity / signed-permutation
                          warm starts return the warm start; 2x2 closed-form
                          angle; Q^T L Q diagonal and Q orthogonal on random SPD
  factor_update ......... the Shampoo chapter's worked example L = G G^T =
                          [[10, 3], [3, 5]]; unrolled EMA sums
  soap_step ............. polar pin: one refreshed step with beta1 = beta2 = 0 is
                          the SVD polar factor U V^T of G; orthogonal
                          equivariance of the whole step; the moments' basis
                          (S4) against unrolled sums over changing bases
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
from scipy.optimize import linear_sum_assignment


@dataclass
class SoapHyper:
    lr: float = 2.8e-3          # [CLEAN-T] Table 6
    beta1: float = 0.95         # [CLEAN-T] Table 6
    beta2: float = 0.95         # [CLEAN-T] Table 6
    shampoo_beta: float = 0.95  # [CLEAN-T] Table 6: EMA coefficient of L and R
    eps: float = 1e-8           # [CLEAN-T] Table 4
    weight_decay: float = 0.1   # [CLEAN-T] Table 4 (S5)
    freq: int = 10              # [CLEAN-T] Table 6: preconditioning frequency f
    bias_correction: bool = True   # S1
    moments: str = "param"      # S4: "param" (Algorithm 4) or "eigen" ([KPOP])

    def refresh(self, t: int) -> bool:
        """[CLEAN-C]: the eigenbases are recomputed after step t when t % f == 0."""
        return self.freq >= 1 and t % self.freq == 0


@dataclass
class SoapState:
    W: np.ndarray
    M: np.ndarray     # first moment (parameter space, or eigenbasis under S4 "eigen")
    V: np.ndarray     # second moment, eigenbasis coordinates
    L: np.ndarray     # m x m factor
    R: np.ndarray     # n x n factor
    QL: np.ndarray
    QR: np.ndarray


def init_state(W: np.ndarray) -> SoapState:
    """S3."""
    m, n = W.shape
    return SoapState(W=np.array(W, dtype=np.float64), M=np.zeros((m, n)), V=np.zeros((m, n)),
                     L=np.zeros((m, m)), R=np.zeros((n, n)), QL=np.eye(m), QR=np.eye(n))


def rotate_in(QL, X, QR):
    """[CLEAN-C] / [KPOP]: coordinates of X in the eigenbasis, Q_L^T X Q_R."""
    return QL.T @ X @ QR


def rotate_out(QL, X, QR):
    """[CLEAN-C] / [KPOP]: back to the parameter space, Q_L X Q_R^T."""
    return QL @ X @ QR.T


def adam_direction(Mr, V, t: int, hp: SoapHyper):
    """S1: the element-wise Adam ratio in the eigenbasis."""
    c1 = 1.0 - hp.beta1 ** t if hp.bias_correction else 1.0
    c2 = 1.0 - hp.beta2 ** t if hp.bias_correction else 1.0
    return (Mr / c1) / (np.sqrt(V / c2) + hp.eps)


def factor_update(L, R, G, beta: float):
    """[CLEAN-C] (after the step): L <- beta L + (1 - beta) G G^T,
    R <- beta R + (1 - beta) G^T G."""
    return beta * L + (1.0 - beta) * (G @ G.T), beta * R + (1.0 - beta) * (G.T @ G)


def eigenvectors(A, Q_prev):
    """S2: eigh of the symmetric part of A, columns matched one-to-one to the
    warm start by largest squared overlap, signs aligned with it."""
    A = 0.5 * (A + A.T)
    _, E = np.linalg.eigh(A)
    overlap = (Q_prev.T @ E) ** 2
    rows, cols = linear_sum_assignment(-overlap)
    Q = np.empty_like(E)
    Q[:, rows] = E[:, cols]
    s = np.sign(np.sum(Q_prev * Q, axis=0))
    s[s == 0] = 1.0
    return Q * s


def offdiag_residual(Q, A) -> float:
    """||off-diagonal of Q^T A Q||_F / ||A||_F (0 for an exact eigenbasis)."""
    B = Q.T @ A @ Q
    den = np.linalg.norm(A)
    off = B - np.diag(np.diag(B))
    return float(np.linalg.norm(off) / (den if den > 0 else 1.0))


def orthogonality(Q) -> float:
    """||Q^T Q - I||_F / sqrt(d)."""
    d = Q.shape[1]
    return float(np.linalg.norm(Q.T @ Q - np.eye(d)) / np.sqrt(d))


@dataclass
class SoapResult:
    state: SoapState
    G_rot: np.ndarray      # G' = Q_L^T G Q_R (bases before the step's refresh)
    M_rot: np.ndarray      # M' (the rotated first moment)
    N_rot: np.ndarray      # N' (the Adam direction in the eigenbasis)
    N: np.ndarray          # Q_L N' Q_R^T
    refreshed: bool


def soap_step(st: SoapState, G: np.ndarray, hp: SoapHyper, t: int, bases=None) -> SoapResult:
    """One step of [CLEAN-C] Algorithm 4 for one matrix, in its order:
    rotate, moments, Adam direction, rotate back, update W, update the
    factors, refresh the eigenbases when t % f == 0.  bases=(QL, QR), if
    given, replaces the refresh's eigenvectors (teacher forcing on a
    computed basis; the factors are still updated)."""
    G = np.asarray(G, dtype=np.float64)
    QL, QR = st.QL, st.QR
    Gr = rotate_in(QL, G, QR)
    if hp.moments == "param":
        M = hp.beta1 * st.M + (1.0 - hp.beta1) * G
        Mr = rotate_in(QL, M, QR)
    elif hp.moments == "eigen":
        M = hp.beta1 * st.M + (1.0 - hp.beta1) * Gr
        Mr = M
    else:
        raise ValueError(hp.moments)
    V = hp.beta2 * st.V + (1.0 - hp.beta2) * Gr * Gr
    Nr = adam_direction(Mr, V, t, hp)
    N = rotate_out(QL, Nr, QR)
    W = (1.0 - hp.lr * hp.weight_decay) * st.W - hp.lr * N
    L, R = factor_update(st.L, st.R, G, hp.shampoo_beta)
    refreshed = hp.refresh(t)
    if refreshed:
        if bases is not None:
            QL, QR = bases
        else:
            QL, QR = eigenvectors(L, QL), eigenvectors(R, QR)
    return SoapResult(SoapState(W, M, V, L, R, np.array(QL), np.array(QR)), Gr, Mr, Nr, N, refreshed)
