"""Plain fp64 CPU oracle for the Online KL Shampoo / Shampoo preconditioner step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or helpers
with the HIP library; the two meet only at seeded inputs.

Every function below follows a passage of the source pages, cited by page
title and section.  Short names used in the citations:

  [OKLS]     "Online KL Shampoo" (project README page), sections "How it works",
             "Hyperparameters", "Batched matrices", "Learning-rate schedule".
  [SHAMPOO]  "Shampoo: 그래디언트 행렬 하나로 두 조각을" (optim-book chapter),
             sections "2 × 3 그래디언트 하나로 손계산" (worked example) and
             "문제 14" (problem 14, exponent and scale).
  [CLEAN]    "Clean: Second-order LLM Training at Linear Memory Cost via
             Nyström Sketching", section 2, equations (2)-(3); Table 6
             (optimizer-specific hyperparameters).
  [MUON]     [SHAMPOO] section "ML에서: 대회 우승과 그다음" (with accumulation
             off, the Shampoo step is the gradient with every singular value
             set to 1; Muon reaches it with matrix products only).

Where the pages leave a step open, the reading taken is named in the
docstring as R1..R16; the list of readings lives with the project's design
notes.  All arithmetic is numpy float64; eigendecompositions use LAPACK
(numpy.linalg.eigh).  Nothing here is blocked, fused or reordered beyond the
definitions.

Parity status of each function (what pins it in the CPU test-suite):
  c_shape ...................... closed forms (square case 1/(2 sqrt n))
  nesterov_scale / momentum .... t=1 gives N=G exactly; Monte-Carlo RMS of N = 1
  factor_update_okls ........... white-Gaussian expectation, equivariance, transpose
  factor_rows / factor_block ... principal blocks of the full updates (both modes)
  factor_update_shampoo ........ worked example L = G G^T = [[10,3],[3,5]]
  inv_root_exact ............... P S P = I, 2x2 closed form, scipy sqrtm on 3x3,
                                 worked example and problem 14 singular values
  ns_coefficients .............. classical Newton-Schulz limit (3/2, -1/2),
                                 equioscillation, grid-search optimality; the
                                 classical table (R4 alternative) converges
                                 quadratically to the eigh root
  ns_spectral / closed form .... matrix iterations (damped, p = 2 and 4) on random SPD
                                 factors; output within the coefficient bound of
                                 (lambda + delta c)^{-1/2} on the design interval
  ns_residual .................. hand-computed classical values on a scalar matrix
                                 (K = 1 and 2); equals the per-eigenvalue recurrence
                                 (eigh) on random SPD factors
  ns_inv_sqrt / ns_inv_quarter . diagonal S reduces to scalar recurrences,
                                 eigen closed form, worked example through NS,
                                 damped isotropic closed form, damped root within
                                 the coefficient bound of eigh's (S + delta c I)^{-1/2}
  whiten / update_weights ...... G=0 step gives W' = (1 - lr wd) W exactly; R6 decay
                                 order: both give decay W for a zero update, decay-after
                                 from W = 0 is decay x the decay-free step; R7 plain
                                 update: the worked example's singular values 1, 1 / 0.5
                                 / 0.1 appear in the weight steps themselves
  eps placement (R1) ........... zero-gradient geometric series (literal) and the
                                 exact fixed point eps I (convex)
  okls_step / shampoo_step ..... orthogonal equivariance, transpose identity,
                                 3-D batch = per-matrix results
  Hyper.refresh (R15) .......... worked example with a refresh period: the singular
                                 values follow the last refresh's accumulation count
  ns_polar / muon_step (R16) ... converges to the SVD polar factor; equals the exact
                                 un-accumulated Shampoo step on the worked example
                                 (singular values 1, 1); 5-step output = the scalar map
                                 on SVD singular values; scale invariance (problem 14),
                                 transpose identity, t = 1 update
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


# ---------------------------------------------------------------------------
# Hyperparameters  ([OKLS] "Hyperparameters": defaults lr 0.09434,
# beta1 0.9684, beta2 0.9482, eps 1e-9, weight_decay 0.0303)
# ---------------------------------------------------------------------------
@dataclass
class Hyper:
    lr: float = 0.09434
    beta1: float = 0.9684
    beta2: float = 0.9482
    eps: float = 1e-9
    weight_decay: float = 0.0303
    lr_peak: float | None = None        # [OKLS] "Learning-rate schedule": the initial lr is kept as lr_peak
    nesterov_var_corr: bool = True      # R5
    ns_steps: int = 10                  # [OKLS] intro: 10-step inverse-root method
    ns_floor: float = 3e-2              # R4: lower end of the design interval for sqrt(lambda / ||S||_F)
                                        # (the fp16 path's; 1e-3 for the fp32-accurate path)
    ns_damping: float = 0.0             # R13: nu; the iteration roots S + (nu/sqrt(d)) ||S||_F I
    root_period: int = 1                # roots refreshed on steps 1, 1 + p, 1 + 2p, ... (R15)
    eps_convex: bool = False            # R1 alternative: OKLS factors get (1-beta2) eps I per update
    decay_after: bool = False           # R6 alternative: decay applied after the update
    shape_scale: bool = True            # R7 alternative (False): the plain update W - lr U, no c_shape
    ns_classical: bool = False          # R4 alternative: the classical step (3/2, -1/2) at every step

    def peak(self) -> float:
        return self.lr if self.lr_peak is None else self.lr_peak

    def coeffs(self):
        """The Newton-Schulz table of this configuration (R4 or its classical alternative)."""
        return ns_coefficients(self.ns_floor, self.ns_steps, self.ns_classical)[0]

    def refresh(self, t: int) -> bool:
        """R15: whether step t (1-based) recomputes the roots.  [OKLS] intro
        refreshes every step (p = 1, no staleness); [SHAMPOO] "Shampoo" and
        [CLEAN] section 2 describe recomputing the roots only every few steps
        and keeping them in between."""
        return self.root_period <= 1 or (t - 1) % self.root_period == 0


# ---------------------------------------------------------------------------
# [OKLS] "How it works": muP shape multiplier c_shape = sqrt(m/n) / (sqrt(m) + sqrt(n)),
# with G in R^{m x n}; m is the number of rows (R3).
# ---------------------------------------------------------------------------
def c_shape(m: int, n: int) -> float:
    return math.sqrt(m / n) / (math.sqrt(m) + math.sqrt(n))


# ---------------------------------------------------------------------------
# [OKLS] intro + "Hyperparameters": Nesterov momentum with variance correction,
# beta1 the momentum EMA coefficient.  The pages give no formula (R5).
# Reading: M_t = beta1 M_{t-1} + (1-beta1) G_t;  N_t = s_t (beta1 M_t + (1-beta1) G_t),
# with s_t = v_t^{-1/2} and v_t the variance of beta1 M_t + (1-beta1) G_t when the
# G_s are independent with unit variance and M_0 = 0.
# ---------------------------------------------------------------------------
def nesterov_scale(beta1: float, t: int, enabled: bool = True) -> float:
    if not enabled:
        return 1.0
    if t < 1:
        raise ValueError("t is 1-based")
    # weight on G_t: beta1 (1-beta1) + (1-beta1) = (1-beta1)(1+beta1)
    v = ((1.0 - beta1) * (1.0 + beta1)) ** 2
    # weights on G_s, s<t: beta1 * (1-beta1) * beta1^(t-s)
    for s in range(1, t):
        v += (beta1 * (1.0 - beta1) * beta1 ** (t - s)) ** 2
    return 1.0 / math.sqrt(v)


def momentum(M: np.ndarray, G: np.ndarray, beta1: float, t: int, var_corr: bool = True):
    """Returns (M_t, N_t) for one step; see nesterov_scale for the reading."""
    M_new = beta1 * M + (1.0 - beta1) * G
    N = nesterov_scale(beta1, t, var_corr) * (beta1 * M_new + (1.0 - beta1) * G)
    return M_new, N


# ---------------------------------------------------------------------------
# [OKLS] "How it works": two-sided KL factor updates using the previous
# preconditioners,
#   S_a <- beta2 S_a + (1-beta2)/n (G P_b)(G P_b)^T
#   S_b <- beta2 S_b + (1-beta2)/m (P_a G)^T (P_a G)
# [OKLS] "Hyperparameters": eps is added during factor initialisation and
# updates (R1: + eps I after every update).  R1's convex alternative keeps
# the update a convex combination, beta2 S + (1-beta2)(X X^T / n + eps I):
# the eps term is weighted by (1-beta2), and eps I is then its fixed point.
# ---------------------------------------------------------------------------
def _eps_term(eps: float, beta2: float, convex: bool) -> float:
    return (1.0 - beta2) * eps if convex else eps


def factor_update_okls(Sa, Sb, Pa, Pb, G, beta2: float, eps: float, eps_convex: bool = False):
    m, n = G.shape
    Xa = G @ Pb
    Xb = Pa @ G
    e = _eps_term(eps, beta2, eps_convex)
    Sa_new = beta2 * Sa + ((1.0 - beta2) / n) * (Xa @ Xa.T) + e * np.eye(m)
    Sb_new = beta2 * Sb + ((1.0 - beta2) / m) * (Xb.T @ Xb) + e * np.eye(n)
    return _sym(Sa_new), _sym(Sb_new)


def factor_rows(G, Pa, Pb, K, side: str, mode: str = "okls"):
    """Rows K of the matrix whose Gram matrix updates one factor: side 'a'
    gives X_a[K] = G[K] P_b, side 'b' gives (P_a G[:, K])^T, the rows K of
    X_b^T (Shampoo, R7: X = G).  Sampled form of the products above."""
    K = np.asarray(K)
    if side == "a":
        return G[K] if mode == "shampoo" else G[K] @ Pb
    return G[:, K].T if mode == "shampoo" else (Pa @ G[:, K]).T


def factor_block(S_KK, X_K, beta2: float, eps: float, den: int, mode: str = "okls", eps_convex: bool = False):
    """Principal block S'[K, K] of a factor update from the rows K of its X:
    (X X^T)[K, K] = X[K] X[K]^T and (eps I)[K, K] = eps I, so the block needs
    nothing else.  OKLS: beta2 S + (1-beta2)/den X X^T + eps I (den = n for
    S_a, m for S_b); Shampoo (R7): S + X X^T + eps I."""
    k = S_KK.shape[0]
    if mode == "shampoo":
        return _sym(S_KK + X_K @ X_K.T + eps * np.eye(k))
    return _sym(beta2 * S_KK + ((1.0 - beta2) / den) * (X_K @ X_K.T) + _eps_term(eps, beta2, eps_convex) * np.eye(k))


# ---------------------------------------------------------------------------
# [CLEAN] eq (2) and [SHAMPOO] worked example: L = sum G G^T, R = sum G^T G.
# R7: the accumulators start at eps I and get + eps I per update (R1).
# ---------------------------------------------------------------------------
def factor_update_shampoo(Sa, Sb, G, eps: float):
    m, n = G.shape
    Sa_new = Sa + G @ G.T + eps * np.eye(m)
    Sb_new = Sb + G.T @ G + eps * np.eye(n)
    return _sym(Sa_new), _sym(Sb_new)


def _sym(S):
    return 0.5 * (S + S.T)


# ---------------------------------------------------------------------------
# Exact inverse p-th roots ([OKLS] "How it works": P = S^{-1/2};
# [CLEAN] eq (3) / [SHAMPOO]: L^{-1/4}, R^{-1/4}).  Principal root of an SPD
# matrix via the symmetric eigendecomposition.
# ---------------------------------------------------------------------------
def cond(S: np.ndarray) -> float:
    """lambda_max / lambda_min of a symmetric matrix (inf if not positive definite)."""
    lam = np.linalg.eigvalsh(_sym(S))
    return float(lam[-1] / lam[0]) if lam[0] > 0 else float("inf")


def inv_root_exact(S: np.ndarray, p: int):
    """Returns (S^{-1/p}, condition number lambda_max / lambda_min)."""
    lam, V = np.linalg.eigh(_sym(S))
    if lam[0] <= 0.0:
        raise np.linalg.LinAlgError("factor is not positive definite")
    P = (V * lam ** (-1.0 / p)) @ V.T
    return _sym(P), float(lam[-1] / lam[0])


# ---------------------------------------------------------------------------
# Coupled Newton-Schulz coefficients (R4).  [OKLS] intro and "How it works":
# a 10-step inverse-root iteration with Chebyshev-optimised coefficients and
# deterministic per-step scales that keep the fp16 inputs in range.  The
# coefficients themselves are not printed; the reading is the per-step minimax
# odd cubic:
#   step k acts on each eigen-direction as  sigma -> sigma (a_k + b_k sigma^2),
#   (a_k, b_k) minimise max |sigma (a + b sigma^2) - 1| over sigma in [l_k, u_k],
#   the minimax error E_k is attained with alternating sign at l_k, at the
#   interior maximum x_k and at u_k (equioscillation of a 2-parameter family).
# Every step but the last is divided by (1 + E_k) so the mapped interval is
# [(1-E_k)/(1+E_k), 1] and no iterate exceeds 1; the last step is left as is so
# the output is centred on 1.
# ---------------------------------------------------------------------------
def _minimax_cubic(lo: float, hi: float):
    # p(x) = a x + b x^3, p(lo) = p(hi) = 1 - E, p(x*) = 1 + E, p'(x*) = 0.
    # p(lo) = p(hi)  =>  a = -b (hi^2 + hi lo + lo^2);  x*^2 = (hi^2 + hi lo + lo^2) / 3
    # p(x*) = -2 b x*^3,  p(lo) = -b lo hi (lo + hi);  p(x*) + p(lo) = 2.
    q = hi * hi + hi * lo + lo * lo
    xs = math.sqrt(q / 3.0)
    b = -2.0 / (2.0 * xs ** 3 + lo * hi * (lo + hi))
    a = -b * q
    err = -2.0 * b * xs ** 3 - 1.0
    return a, b, err


def ns_coefficients(floor: float = 1e-3, steps: int = 10, classical: bool = False):
    """List of (a_k, b_k) for k = 0..steps-1 and the final interval half-width.
    classical: the textbook Newton-Schulz step T = (3 I - Z Y) / 2, i.e.
    sigma -> sigma (3 - sigma^2) / 2, at every step (R4's plainest
    alternative); no interval is designed, so the half-width is None."""
    if classical:
        return [(1.5, -0.5)] * steps, None
    lo, hi = floor, 1.0
    coeffs = []
    err = 0.0
    for k in range(steps):
        a, b, err = _minimax_cubic(lo, hi)
        if k < steps - 1:
            a, b = a / (1.0 + err), b / (1.0 + err)
            lo, hi = (1.0 - err) / (1.0 + err), 1.0
        coeffs.append((a, b))
    return coeffs, err


# ---------------------------------------------------------------------------
# Coupled Newton-Schulz inverse square root in fp64 ([OKLS] "How it works":
# roots evaluated by the coupled iteration; intro: 10 steps, 27 GEMMs).
#   Y_0 = S / c with c = ||S||_F (so the spectrum lies in (0, 1]), Z_0 = I,
#   T_k = a_k I + b_k Z_k Y_k,  Y_{k+1} = Y_k T_k,  Z_{k+1} = T_k Z_k.
#   Z_K -> (S/c)^{-1/2}, Y_K -> (S/c)^{1/2};  P = Z_K / sqrt(c).
# This is the iteration itself (the GPU's algorithm in exact-ish arithmetic);
# the exact eigh root above is the method's target.
# ---------------------------------------------------------------------------
#
# R13 (damping): the pages fix eps = 1e-9 absolutely, far below what fp16
# inputs resolve; rounding then leaves eigenvalues of the normalised factor
# slightly negative and the cubic step amplifies them without bound.  The
# iteration is therefore run on the shifted matrix S + delta c I with
# delta = nu / sqrt(d) (the size of the rounding perturbation of a
# Frobenius-normalised d x d matrix scales as 1/sqrt(d)), normalised by
# c' = c (1 + delta) so its spectrum stays in (0, 1].  nu = 0 is the plain
# iteration.
def ns_inv_sqrt(S: np.ndarray, coeffs, nu: float = 0.0):
    """Returns (P, R): estimates of (S + delta c I)^{-1/2} and (S + delta c I)^{1/2}
    after len(coeffs) steps, delta = nu / sqrt(d)."""
    d = S.shape[0]
    eye = np.eye(d)
    delta = nu / math.sqrt(d)
    c = float(np.linalg.norm(S)) * (1.0 + delta)
    Y = (S + (delta * c / (1.0 + delta)) * eye) / c
    Z = eye.copy()
    for a, b in coeffs:
        T = a * eye + b * (Z @ Y)
        Y, Z = Y @ T, T @ Z
    return Z / math.sqrt(c), Y * math.sqrt(c)


def ns_residual(S: np.ndarray, coeffs, nu: float = 0.0) -> float:
    """Convergence diagnostic of the iteration above: ||Z_{K-1} Y_{K-1} - I||_F,
    the product the last step's T_{K-1} = a I + b Z_{K-1} Y_{K-1} is formed
    from (K = len(coeffs); for K = 1 that is Z_0 Y_0 = Y_0).  Z_k Y_k -> I as
    the iteration converges."""
    d = S.shape[0]
    eye = np.eye(d)
    delta = nu / math.sqrt(d)
    c = float(np.linalg.norm(S)) * (1.0 + delta)
    Y = (S + (delta * c / (1.0 + delta)) * eye) / c
    Z = eye.copy()
    ZY = Z @ Y
    for a, b in coeffs:
        ZY = Z @ Y
        T = a * eye + b * ZY
        Y, Z = Y @ T, T @ Z
    return float(np.linalg.norm(ZY - eye))


def ns_residual_spectral(lam: np.ndarray, coeffs, nu: float = 0.0) -> float:
    """ns_residual through the eigenvalues (the per-direction recurrence of
    ns_spectral): in each eigen-direction Z_k Y_k = sigma_k^2, so the residual
    is (sum over directions of (sigma_{K-1}^2 - 1)^2)^1/2."""
    lam = np.asarray(lam, dtype=np.float64)
    d = lam.size
    delta = nu / math.sqrt(d)
    c = float(np.linalg.norm(lam))
    s = np.sqrt((lam + delta * c) / (c * (1.0 + delta)))
    for a, b in coeffs[:-1]:
        s = s * (a + b * s * s)
    return float(np.sqrt(np.sum((s * s - 1.0) ** 2)))


def ns_inv_quarter(S: np.ndarray, coeffs, nu: float = 0.0):
    """S^{-1/4} = (S^{-1/2})^{1/2} as two chained iterations (R8): the first
    chain's Z output P1 = S^{-1/2}, then the square root of sym(P1) from the
    second chain's Y output."""
    P1, _ = ns_inv_sqrt(S, coeffs, nu)
    _, P = ns_inv_sqrt(_sym(P1), coeffs, nu)
    return P


def ns_spectral(lam: np.ndarray, coeffs, nu: float = 0.0, p: int = 2, out: str = "inv"):
    """Exact-arithmetic output of the damped coupled iteration(s) on a
    symmetric matrix with eigenvalues `lam`, one value per eigen-direction.

    One chain on S (dimension d = len(lam), c = ||S||_F = ||lam||_2,
    delta = nu / sqrt(d), c' = c (1 + delta)) starts from y = (lam + delta c) / c'.
    Every matrix of the iteration is a polynomial in Y_0, so in each
    eigen-direction Z_k Y_k = sigma_k^2 with sigma_0 = sqrt(y) and
    sigma_{k+1} = sigma_k (a_k + b_k sigma_k^2); Z_K = sigma_K / sqrt(y) and
    Y_K = sigma_K sqrt(y).  Hence the chain returns
        P = Z_K / sqrt(c') = sigma_K / sqrt(lam + delta c)    (out='inv')
        R = Y_K sqrt(c')  = sigma_K sqrt(lam + delta c)      (out='sqrt').
    p = 2 returns that chain's output; p = 4 (R8) runs a second chain on
    the first chain's P eigenvalues and returns its R.

    The factor is positive semidefinite (outer products plus eps I), so an
    eigenvalue below zero is the eigensolver's rounding and is taken as zero.
    The ratio t_k = sigma_k / sigma_0 runs through the same recurrence:
    P = t_K / sqrt(c') equals sigma_K / sqrt(lam + delta c) wherever that is
    defined, and is the iteration's limit on a zero eigenvalue."""
    lam = np.asarray(lam, dtype=np.float64)
    d = lam.size
    delta = nu / math.sqrt(d)
    c = float(np.linalg.norm(lam))
    cp = c * (1.0 + delta)
    shifted = np.maximum(lam + delta * c, 0.0)
    s = np.sqrt(shifted / cp)
    t = np.ones_like(s)
    for a, b in coeffs:
        g = a + b * s * s
        s = s * g
        t = t * g
    if p == 2:
        return t / math.sqrt(cp) if out == "inv" else s * np.sqrt(shifted)
    if p == 4:
        return ns_spectral(t / math.sqrt(cp), coeffs, nu, 2, "sqrt")
    raise ValueError("p must be 2 or 4")


def ns_eigen_closed_form(S: np.ndarray, coeffs, p: int = 2, nu: float = 0.0):
    """Exact-arithmetic output of ns_inv_sqrt (p = 2) or ns_inv_quarter (p = 4)
    through the eigendecomposition: P = V diag(ns_spectral(lambda)) V^T.
    Used as a diagnostic and a pin, and where the matrix iteration in fp64
    would take too long."""
    lam, V = np.linalg.eigh(_sym(S))
    return (V * ns_spectral(lam, coeffs, nu, p)) @ V.T


# ---------------------------------------------------------------------------
# [OKLS] "How it works": U = P_a N P_b; c_shape scaling.
# R6 (AdamC, [OKLS] "Learning-rate schedule"/"Hyperparameters"): decoupled decay
# with the factor lr / lr_peak, applied to the previous weights.
# ---------------------------------------------------------------------------
def whiten(Pa, N, Pb):
    return Pa @ N @ Pb


def update_weights(W, U, lr: float, lr_peak: float, wd: float, shape=None, decay_after: bool = False,
                   shape_scale: bool = True):
    """shape: (m, n) of the whole matrix when W and U hold only some of its rows.
    R6: the decay multiplies the previous weights (decay_after: the updated
    ones, decay (W - lr c U)).  R7's alternative (shape_scale False) is the
    original Shampoo update, the step without the muP multiplier."""
    m, n = W.shape if shape is None else shape
    decay = 1.0 - lr * wd * (lr / lr_peak)
    c = c_shape(m, n) if shape_scale else 1.0
    if decay_after:
        return decay * (W - lr * c * U)
    return decay * W - lr * c * U


# ---------------------------------------------------------------------------
# State and full steps.
# ---------------------------------------------------------------------------
@dataclass
class MatState:
    W: np.ndarray
    M: np.ndarray
    Sa: np.ndarray
    Sb: np.ndarray
    Pa: np.ndarray
    Pb: np.ndarray


def init_state(W: np.ndarray, eps: float) -> MatState:
    """[OKLS] "Hyperparameters": eps added at factor initialisation (S_0 = eps I);
    R2: P_0 = I; momentum starts at zero."""
    m, n = W.shape
    return MatState(W=np.array(W, dtype=np.float64), M=np.zeros((m, n)),
                    Sa=eps * np.eye(m), Sb=eps * np.eye(n), Pa=np.eye(m), Pb=np.eye(n))


@dataclass
class StepResult:
    state: MatState
    N: np.ndarray
    U: np.ndarray
    Pa_ns: np.ndarray | None = None
    Pb_ns: np.ndarray | None = None
    kappa_a: float = 0.0
    kappa_b: float = 0.0
    extra: dict = field(default_factory=dict)


def okls_step(st: MatState, G: np.ndarray, hp: Hyper, t: int, root: str = "exact") -> StepResult:
    """One OKLS step for one matrix ([OKLS] "How it works", in its order):
    factors with the previous P, fresh roots, Nesterov momentum, two-sided
    whitening, c_shape-scaled update with AdamC decay.
    root='exact' uses eigh roots (the method's target); root='ns' uses the
    coupled Newton-Schulz iteration in fp64.  Both are always reported."""
    G = np.asarray(G, dtype=np.float64)
    Sa, Sb = factor_update_okls(st.Sa, st.Sb, st.Pa, st.Pb, G, hp.beta2, hp.eps, hp.eps_convex)
    if not hp.refresh(t):          # R15: the previous roots are kept
        Pa, Pb = st.Pa, st.Pb
        Pa_ns, Pb_ns, ka, kb = Pa, Pb, float("nan"), float("nan")
    else:
        coeffs = hp.coeffs()
        Pa_ns, _ = ns_inv_sqrt(Sa, coeffs, hp.ns_damping)
        Pb_ns, _ = ns_inv_sqrt(Sb, coeffs, hp.ns_damping)
        if root == "exact":
            (Pa, ka), (Pb, kb) = inv_root_exact(Sa, 2), inv_root_exact(Sb, 2)
        else:
            Pa, Pb, ka, kb = Pa_ns, Pb_ns, cond(Sa), cond(Sb)
    M, N = momentum(st.M, G, hp.beta1, t, hp.nesterov_var_corr)
    U = whiten(Pa, N, Pb)
    W = update_weights(st.W, U, hp.lr, hp.peak(), hp.weight_decay, decay_after=hp.decay_after,
                       shape_scale=hp.shape_scale)
    return StepResult(MatState(W, M, Sa, Sb, Pa, Pb), N, U, Pa_ns, Pb_ns, ka, kb)


def shampoo_step(st: MatState, G: np.ndarray, hp: Hyper, t: int, root: str = "exact") -> StepResult:
    """Classic Shampoo mode (R7): sums G G^T and G^T G, P = S^{-1/4}
    ([CLEAN] eq (2)-(3), [SHAMPOO] worked example); momentum, c_shape and
    decoupled decay as in OKLS."""
    G = np.asarray(G, dtype=np.float64)
    Sa, Sb = factor_update_shampoo(st.Sa, st.Sb, G, hp.eps)
    if not hp.refresh(t):          # R15: the previous roots are kept
        Pa, Pb = st.Pa, st.Pb
        Pa_ns, Pb_ns, ka, kb = Pa, Pb, float("nan"), float("nan")
    else:
        coeffs = hp.coeffs()
        Pa_ns = ns_inv_quarter(Sa, coeffs, hp.ns_damping)
        Pb_ns = ns_inv_quarter(Sb, coeffs, hp.ns_damping)
        if root == "exact":
            (Pa, ka), (Pb, kb) = inv_root_exact(Sa, 4), inv_root_exact(Sb, 4)
        else:
            Pa, Pb, ka, kb = Pa_ns, Pb_ns, cond(Sa), cond(Sb)
    M, N = momentum(st.M, G, hp.beta1, t, hp.nesterov_var_corr)
    U = whiten(Pa, N, Pb)
    W = update_weights(st.W, U, hp.lr, hp.peak(), hp.weight_decay, decay_after=hp.decay_after,
                       shape_scale=hp.shape_scale)
    return StepResult(MatState(W, M, Sa, Sb, Pa, Pb), N, U, Pa_ns, Pb_ns, ka, kb)


# ---------------------------------------------------------------------------
# Muon ([MUON]; [CLEAN] Table 6: Nesterov momentum, 5 Newton-Schulz iterations).
# R16: the iteration X <- a_k X + b_k (X X^T) X maps every singular value by
# sigma (a_k + b_k sigma^2), the scalar map of the coupled inverse-root
# iteration, so it takes the same minimax table (R4) on [l_0, 1]; the Muon
# configuration is 5 steps with l_0 = 1e-2 (final half-width 0.156).  The
# start X_0 = N / ||N N^T||_F^{1/2} puts every singular value in (0, 1]
# (||N N^T||_F = (sum sigma^4)^{1/2} >= sigma_max^2); it is the scaling the
# OKLS chain applies to S = G G^T-like factors.  Momentum, c_shape and the
# decoupled decay are those of the OKLS step.
# ---------------------------------------------------------------------------
def muon_hyper(**kw) -> Hyper:
    """The Muon configuration of R16 (5 steps, l_0 = 1e-2) on top of Hyper's defaults."""
    kw.setdefault("ns_steps", 5)
    kw.setdefault("ns_floor", 1e-2)
    return Hyper(**kw)


def ns_polar(N: np.ndarray, coeffs) -> np.ndarray:
    """The R16 iteration on N; the Gram of the smaller side is formed
    ((X X^T) X and X (X^T X) are the same matrix)."""
    N = np.asarray(N, dtype=np.float64)
    wide = N.shape[0] <= N.shape[1]
    gram = N @ N.T if wide else N.T @ N
    X = N / math.sqrt(float(np.linalg.norm(gram)))
    for a, b in coeffs:
        X = a * X + b * ((X @ X.T) @ X if wide else X @ (X.T @ X))
    return X


def muon_step(st: MatState, G: np.ndarray, hp: Hyper, t: int, root: str = "ns") -> StepResult:
    """One Muon step (R16): Nesterov momentum (R5), N orthogonalised by the
    polar iteration, c_shape-scaled update with the decoupled decay (R6).
    The factors and roots of the state are neither used nor changed.
    root='exact' updates with the SVD polar factor U V^T (the method's
    target) instead of the iteration's result; both are always computed and
    the iteration's is in extra["U_ns"]."""
    G = np.asarray(G, dtype=np.float64)
    M, N = momentum(st.M, G, hp.beta1, t, hp.nesterov_var_corr)
    coeffs = hp.coeffs()
    U_ns = ns_polar(N, coeffs)
    U = U_ns
    if root == "exact":
        u, _, vt = np.linalg.svd(N, full_matrices=False)
        U = u @ vt
    W = update_weights(st.W, U, hp.lr, hp.peak(), hp.weight_decay, decay_after=hp.decay_after,
                       shape_scale=hp.shape_scale)
    return StepResult(MatState(W, M, st.Sa, st.Sb, st.Pa, st.Pb), N, U, st.Pa, st.Pb, float("nan"), float("nan"),
                      extra={"U_ns": U_ns})


def step(st: MatState, G, hp: Hyper, t: int, mode: str = "okls", root: str = "exact") -> StepResult:
    if mode == "okls":
        return okls_step(st, G, hp, t, root)
    if mode == "shampoo":
        return shampoo_step(st, G, hp, t, root)
    if mode == "muon":
        return muon_step(st, G, hp, t, root)
    raise ValueError(mode)


def step_batched(states, Gs, hp: Hyper, t: int, mode: str = "okls", root: str = "exact"):
    """[OKLS] "Batched matrices": a 3-D parameter (N, m, n) is N independent
    matrices sharing the hyperparameters."""
    return [step(s, g, hp, t, mode, root) for s, g in zip(states, Gs)]


def rel_frob(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))
