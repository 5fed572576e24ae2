"""Seeded synthetic inputs for the five preconditioner-step workloads.

This module holds input generation only (shapes, seeds, value
distributions); none of the optimizer's arithmetic lives here.  Both the
HIP path's tests/benchmark and the CPU oracle draw their inputs from it.

The workloads follow the transformer shapes the optimizer is meant for
(the project README of "Online KL Shampoo" lists q, k, v, o, gate, up and
down projections as the matrices it preconditions) at five sizes:

  c1  one 128x256 fp32 matrix, gradients i.i.d. N(0,1) drawn from seed 0 in
      step order; the small case the oracle finishes in seconds.
  c2  one transformer block at d=1024: q,k,v,o 1024x1024, gate/up 2816x1024,
      down 1024x2816; bf16 gradients 0.02 * N(0,1) with a per-row scale drawn
      once per matrix, log-uniform on [0.1, 10].
  c3  24 layers of the 1.2B-class block: 4x 2048x2048, 2x 5632x2048,
      1x 2048x5632; fp32 gradients 0.02 * (sqrt(0.9) L + sqrt(0.1) Z) with
      L = A C B^T a rank-32 part normalised to unit RMS (A, B fixed per
      matrix, C fresh per step) and Z i.i.d. N(0,1).
  c4  32 layers of 4096x4096 (x4), 11008x4096 (x2), 4096x11008 (x1);
      fp32 gradients i.i.d. N(0, 1e-3^2); classic Shampoo mode.
  c5  one layer of 5120x5120 (x4), 13824x5120 (x2), 5120x13824 (x1);
      gradients A Z B with Z i.i.d. N(0,1), A = Q_L diag(s_A), B = diag(s_B) Q_R^T,
      Q dense random orthogonal (RandomOrthogonal), s log-spaced on [1e-3, 1]
      (endpoints included) in random order.

Seeds: every draw comes from numpy's default_rng(SeedSequence([cfg, group,
matrix, t, stream])) except c1, which uses default_rng(0) in step order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

CFG_IDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


@dataclass
class Workload:
    name: str
    groups: list            # list of (m, n, batch)
    mode: str               # "okls" or "shampoo"
    grad: str               # generator kind
    grad_dtype: str         # "f32" or "bf16"
    steps: int
    parity_steps: tuple
    hyper: dict = field(default_factory=dict)

    @property
    def n_matrices(self) -> int:
        return sum(b for _, _, b in self.groups)

    @property
    def n_params(self) -> int:
        return sum(m * n * b for m, n, b in self.groups)


def _block(d, f, layers):
    return [(d, d, 4 * layers), (f, d, 2 * layers), (d, f, 1 * layers)]


WORKLOADS = {
    "c1": Workload("c1", [(128, 256, 1)], "okls", "gauss1", "f32", 20, tuple(range(1, 21))),
    "c2": Workload("c2", _block(1024, 2816, 1), "okls", "rowscaled", "bf16", 100, (1, 2, 5, 10, 25, 50, 100)),
    "c3": Workload("c3", _block(2048, 5632, 24), "okls", "lowrank", "f32", 10, (1, 2, 10)),
    "c4": Workload("c4", _block(4096, 11008, 32), "shampoo", "gauss1e-3", "f32", 5, (1, 2, 5)),
    "c5": Workload("c5", _block(5120, 13824, 1), "okls", "illcond", "f32", 5, (1, 2, 5)),
}


def workload(name: str, layers: int | None = None) -> Workload:
    """Returns the named workload; `layers` overrides the layer count of the
    multi-layer workloads (same shapes, fewer copies)."""
    w = WORKLOADS[name]
    if layers is None or name not in ("c3", "c4"):
        return w
    d, f = (2048, 5632) if name == "c3" else (4096, 11008)
    return Workload(w.name, _block(d, f, layers), w.mode, w.grad, w.grad_dtype, w.steps, w.parity_steps, dict(w.hyper))


def _rng(cfg: str, group: int, mat: int, t: int, stream: int = 0):
    return np.random.default_rng(np.random.SeedSequence([CFG_IDS[cfg], group, mat, t, stream]))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32
    values that are exactly representable in bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(x)
    out = r.view(np.float32).copy()
    out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


class C1Stream:
    """c1's gradients come from one generator, seed 0, in step order."""

    def __init__(self):
        self.rng = np.random.default_rng(0)
        self.t = 0
        self.cache = {}

    def get(self, t: int) -> np.ndarray:
        while self.t < t:
            self.t += 1
            self.cache[self.t] = self.rng.standard_normal((128, 256)).astype(np.float32)
        return self.cache[t]


_C1 = None
_FIXED = {}


class RandomOrthogonal:
    """A dense random orthogonal d x d matrix that is applied in O(d log d)
    instead of being stored: two rounds of Q_r = P_r D_r C E_r, with C the
    orthonormal DCT-II, D_r and E_r random sign diagonals and P_r a random
    row permutation.  Every column has full support (no structure aligned
    with the coordinate axes), so factors built from it are dense."""

    def __init__(self, rng, d: int, rounds: int = 2):
        self.d = d
        self.stages = [(rng.permutation(d), rng.choice([-1.0, 1.0], size=d), rng.choice([-1.0, 1.0], size=d))
                       for _ in range(rounds)]

    @staticmethod
    def _bcast(v, Y, axis):
        return v if Y.ndim == 1 else (v[:, None] if axis == 0 else v[None, :])

    def apply(self, X: np.ndarray, axis: int = 0) -> np.ndarray:
        """Q @ X (axis 0) or X @ Q^T (axis 1, Q applied to every row) for X of
        shape (d,), (d, k) or (k, d); works on a copy, in place."""
        import scipy.fft
        Y = np.array(X, dtype=np.float64, copy=True)
        buf = np.empty_like(Y)
        for perm, dsign, esign in self.stages:
            Y *= self._bcast(esign, Y, axis)
            Y = scipy.fft.dct(Y, type=2, norm="ortho", axis=axis, workers=-1, overwrite_x=True)
            Y *= self._bcast(dsign, Y, axis)
            np.take(Y, perm, axis=axis, out=buf)
            Y, buf = buf, Y
        return Y

    def apply_t(self, X: np.ndarray) -> np.ndarray:
        """Q^T @ X; works on a copy, in place."""
        import scipy.fft
        Y = np.array(X, dtype=np.float64, copy=True)
        buf = np.empty_like(Y)
        for perm, dsign, esign in reversed(self.stages):
            buf[perm] = Y
            Y, buf = buf, Y
            Y *= self._bcast(dsign, Y, 0)
            Y = scipy.fft.idct(Y, type=2, norm="ortho", axis=0, workers=-1, overwrite_x=True)
            Y *= self._bcast(esign, Y, 0)
        return Y

    def rows(self, idx) -> np.ndarray:
        """Rows idx of Q, shape (len(idx), d)."""
        E = np.zeros((self.d, len(idx)))
        E[np.asarray(idx), np.arange(len(idx))] = 1.0
        return self.apply_t(E).T


def symmetric_from_spectrum(Q: RandomOrthogonal, v: np.ndarray, rows=None) -> np.ndarray:
    """Q diag(v) Q^T in fp64 (exactly symmetrised), or only its rows `rows`."""
    v = np.asarray(v, dtype=np.float64)
    if rows is not None:
        R = Q.rows(rows)                      # Q[rows, :]
        return Q.apply(R * v, axis=1)         # Q[rows] diag(v) Q^T
    A = Q.apply(np.diag(v))                   # Q diag(v)
    A = Q.apply(A, axis=1)                    # Q diag(v) Q^T
    A += A.T.copy()
    A *= 0.5
    return A


def spectral_factor(cfg: str, group: int, mat: int, side: int, d: int, kappa: float, lam_max: float):
    """Known-spectrum factor state for the full-size parity checks: the
    eigenvalues are log-uniform on [lam_max / kappa, lam_max] (both ends
    included), the eigenvectors the columns of a RandomOrthogonal.  Returns
    (Q, lam)."""
    rng = _rng(cfg, group, mat, 0, 10 + side)
    lam = lam_max * np.exp(rng.uniform(-math.log(kappa), 0.0, size=d))
    lam[:2] = (lam_max, lam_max / kappa)
    rng.shuffle(lam)
    return RandomOrthogonal(rng, d), lam


def device_filler(scale: float, shape, seed: int, dtype=None):
    """Gaussian filler gradients generated on cuda:0 by torch's own seeded
    generator: scale * N(0, 1).  The full-size checks use them for the
    matrices they do not sample, so that every launch runs at its real size
    without generating billions of values on the host."""
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, device="cuda:0", dtype=torch.float32) * scale
    return x if dtype is None else x.to(dtype)


def device_lowrank(shape, seed_fixed: int, seed_t: int, scale: float = 0.02, rank: int = 32):
    """The low-rank workload's recipe generated on cuda:0 (torch's seeded
    generator) for a whole (b, m, n) group: per matrix
    scale * (sqrt(0.9) L + sqrt(0.1) Z), L = A C B^T normalised to unit RMS,
    with A (m x rank) and B (n x rank) Gaussian fixed by seed_fixed and C
    (rank x rank) and Z fresh from seed_t.  The benchmark uses it for the
    1.2B-class workload, whose host recipe takes minutes per step."""
    import torch
    b, m, n = shape
    gf = torch.Generator(device="cuda:0")
    gf.manual_seed(seed_fixed)
    A = torch.randn(b, m, rank, generator=gf, device="cuda:0")
    B = torch.randn(b, n, rank, generator=gf, device="cuda:0")
    gt = torch.Generator(device="cuda:0")
    gt.manual_seed(seed_t)
    C = torch.randn(b, rank, rank, generator=gt, device="cuda:0")
    L = torch.bmm(torch.bmm(A, C), B.transpose(1, 2).contiguous())
    L = L / torch.sqrt(torch.mean(L * L, dim=(1, 2), keepdim=True))
    Z = torch.randn(b, m, n, generator=gt, device="cuda:0")
    return scale * (math.sqrt(0.9) * L + math.sqrt(0.1) * Z)


def gradient(w: Workload, group: int, mat: int, t: int) -> np.ndarray:
    """fp32 array (m, n) holding the gradient of matrix `mat` of shape group
    `group` at step t (1-based).  bf16 workloads return bf16-representable
    values."""
    global _C1
    m, n, _ = w.groups[group]
    if w.grad == "gauss1":
        if w.name == "c1":
            if _C1 is None:
                _C1 = C1Stream()
            return _C1.get(t)
        return _rng(w.name, group, mat, t).standard_normal((m, n)).astype(np.float32)
    if w.grad == "rowscaled":
        r = np.exp(_rng(w.name, group, mat, 0, 1).uniform(math.log(0.1), math.log(10.0), size=(m, 1)))
        z = _rng(w.name, group, mat, t).standard_normal((m, n))
        g = (0.02 * z * r).astype(np.float32)
        return round_to_bf16(g) if w.grad_dtype == "bf16" else g
    if w.grad == "lowrank":
        key = (w.name, group, mat)
        if key not in _FIXED:
            fr = _rng(w.name, group, mat, 0, 1)
            _FIXED[key] = (fr.standard_normal((m, 32)), fr.standard_normal((n, 32)))
        A, B = _FIXED[key]
        r = _rng(w.name, group, mat, t)
        C = r.standard_normal((32, 32))
        L = (A @ C) @ B.T
        L /= math.sqrt(float(np.mean(L * L)))
        Z = r.standard_normal((m, n))
        return (0.02 * (math.sqrt(0.9) * L + math.sqrt(0.1) * Z)).astype(np.float32)
    if w.grad == "gauss1e-3":
        return (1e-3 * _rng(w.name, group, mat, t).standard_normal((m, n))).astype(np.float32)
    if w.grad == "illcond":
        key = (w.name, group, mat)
        if key not in _FIXED:
            fr = _rng(w.name, group, mat, 0, 1)
            sA = np.exp(np.linspace(math.log(1e-3), 0.0, m))
            sB = np.exp(np.linspace(math.log(1e-3), 0.0, n))
            fr.shuffle(sA)
            fr.shuffle(sB)
            _FIXED[key] = (RandomOrthogonal(fr, m), sA, sB, RandomOrthogonal(fr, n))
        QL, sA, sB, QR = _FIXED[key]
        Z = _rng(w.name, group, mat, t).standard_normal((m, n))
        # G = A Z B with A = Q_L diag(sA), B = diag(sB) Q_R^T
        Z *= sA[:, None]
        Y = QL.apply(Z)
        Y *= sB
        return QR.apply(Y, axis=1).astype(np.float32)
    raise ValueError(w.grad)


def initial_weights(w: Workload, group: int, mat: int, sigma_star: float = 0.07539) -> np.ndarray:
    """Spectral-muP Gaussian initial weights (the README's "Weight
    initialization" recipe): std = sigma* sqrt(n_out/n_in) / (sqrt(n_in) + sqrt(n_out)),
    with W of shape (n_out, n_in) = (m, n)."""
    m, n, _ = w.groups[group]
    std = sigma_star * math.sqrt(m / n) / (math.sqrt(n) + math.sqrt(m))
    return (std * _rng(w.name, group, mat, 0, 2).standard_normal((m, n))).astype(np.float32)


def reset_caches():
    global _C1
    _C1 = None
    _FIXED.clear()
