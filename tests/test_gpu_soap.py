"""GPU parity of the eigenbasis-Adam (SOAP) mode against the fp64 oracle
(oracle/soap_oracle.py), through the C ABI.

Teacher forcing: each step starts the oracle from the GPU's state before the
step and compares the state after it.  On refresh steps the oracle takes the
GPU's new bases (an eigenbasis is not unique where eigenvalues repeat, and
its column order follows the warm start); the bases themselves are checked
by what defines them: orthogonality, Q^T S Q diagonal (its off-diagonal
Frobenius norm against ||S||_F) and its diagonal equal to S's eigenvalues.

Tolerances.  The fp32-accurate path (split-fp16 products, fp32 Jacobi)
carries fp32 rounding: ~1e-6 relative in the products, the Jacobi stop at
2e-6 and a basis orthogonal to ~1e-5.  The fp16 path rounds the operands of
every product to 11 bits: ~1e-3 relative in G', M', S and Q^T S Q.  The
Adam direction is a ratio per element, so its relative error is that of M'
plus half that of V where |M'| and sqrt(V) stand well above eps; the
gradients here are Gaussian, whose rotated entries all do.

The oracle's polar-factor pin (a refreshed step with no averaging gives
U V^T) is not repeated here: it needs G' to vanish off its singular-value
pattern, and a computed eigenbasis leaves there entries of the size of its
error times ||G|| (in fp32, ~1e-6 ||S|| / gap), which the Adam ratio maps to
values near +-1 once they exceed eps.  The comparison with the oracle is
therefore made on the GPU's own bases (teacher forcing), where it is exact
up to rounding.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.linalg

from oracle import soap_oracle as S

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _make(groups, precision, grad_dtype="f32", **cfg):
    torch = _torch()
    from kronecker_factored_second_amd import okls
    dev = torch.device("cuda:0")
    params = [torch.zeros(b, m, n, device=dev) for (m, n, b) in groups]
    gdt = {"f32": torch.float32, "bf16": torch.bfloat16}[grad_dtype]
    opt = okls.OKLS(params, mode="soap", precision=precision, grad_dtype=gdt, **cfg)
    return opt, params


def _hyper(opt, lr):
    c = opt.cfg
    return S.SoapHyper(lr=lr, beta1=float(np.float32(c.beta1)), beta2=float(np.float32(c.beta2)),
                       shampoo_beta=float(np.float32(c.soap_beta)), eps=float(np.float32(c.eps)),
                       weight_decay=float(np.float32(c.weight_decay)), freq=int(c.precond_freq),
                       bias_correction=bool(c.bias_correction), moments="eigen" if c.soap_moments else "param")


def _snap(opt, gi, i):
    s = opt.state[gi]
    f = lambda t: t[i].detach().double().cpu().numpy()
    return S.SoapState(W=f(opt.params[gi]), M=f(s["M"]), V=f(s["V"]), L=f(s["Sa"]), R=f(s["Sb"]),
                       QL=f(s["Pa"]), QR=f(s["Pb"]))


def _rel(x, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _eig_err(Q, A):
    """Largest gap between the diagonal of Q^T A Q and A's eigenvalues (sorted), over ||A||_F."""
    d = np.sort(np.diag(Q.T @ A @ Q))
    lam = np.linalg.eigvalsh(0.5 * (A + A.T))
    den = np.linalg.norm(A)
    return float(np.max(np.abs(d - lam)) / (den if den > 0 else 1.0))


TOL = {
    "fp32": dict(W=2e-4, M=1e-6, V=2e-5, F=2e-5, orth=2e-5, res=2e-5, eig=2e-5),
    "fp16": dict(W=3e-2, M=1e-6, V=1e-2, F=5e-3, orth=2e-5, res=5e-3, eig=5e-3),
}


def _grad(rng, gi, shape, dtype):
    G = rng.standard_normal(shape)
    if dtype == "bf16":      # the values the GPU reads
        G = _torch().tensor(G, dtype=_torch().float32).to(_torch().bfloat16).double().numpy()
    return G


def _run(groups, precision, steps, grad_dtype="f32", lr=0.01, seed=0, **cfg):
    torch = _torch()
    opt, params = _make(groups, precision, grad_dtype, lr=lr, **cfg)
    hp = _hyper(opt, lr)
    tol = dict(TOL[precision])
    if cfg.get("soap_moments"):   # M holds rotated gradients: the products' error, like V's
        tol["M"] = tol["V"]
    rng = np.random.default_rng(seed)
    worst = {}
    for t in range(1, steps + 1):
        Gs = [np.stack([_grad(rng, gi, (m, n), grad_dtype) for _ in range(b)]) for gi, (m, n, b) in enumerate(groups)]
        before = [[_snap(opt, gi, i) for i in range(b)] for gi, (m, n, b) in enumerate(groups)]
        tdt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
        opt.step(grads=[torch.tensor(G, dtype=torch.float32, device="cuda:0").to(tdt) for G in Gs])
        torch.cuda.synchronize()
        for gi, (m, n, b) in enumerate(groups):
            for i in range(b):
                got = _snap(opt, gi, i)
                r = S.soap_step(before[gi][i], Gs[gi][i], hp, t, bases=(got.QL, got.QR))
                e = dict(W=_rel(got.W - before[gi][i].W, r.state.W - before[gi][i].W),
                         M=_rel(got.M, r.state.M), V=_rel(got.V, r.state.V),
                         F=max(_rel(got.L, r.state.L), _rel(got.R, r.state.R)))
                if r.refreshed:
                    e["orth"] = max(S.orthogonality(got.QL), S.orthogonality(got.QR))
                    e["res"] = max(S.offdiag_residual(got.QL, r.state.L), S.offdiag_residual(got.QR, r.state.R))
                    e["eig"] = max(_eig_err(got.QL, r.state.L), _eig_err(got.QR, r.state.R))
                else:
                    assert np.array_equal(got.QL, before[gi][i].QL) and np.array_equal(got.QR, before[gi][i].QR), \
                        f"t={t}: the bases changed on a step that keeps them"
                print(f"t={t} group={gi} i={i} refresh={r.refreshed} " +
                      " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
                for k, v in e.items():
                    assert v <= tol[k], f"t={t} group {gi} matrix {i}: {k} error {v:.3e} > {tol[k]:.1e}"
                    worst[k] = max(worst.get(k, 0.0), v)
    assert opt.check_finite()
    return worst


@pytest.mark.parametrize("precision", ["fp32", "fp16"])
@pytest.mark.parametrize("moments", [0, 1])
def test_soap_teacher_forced_ragged(precision, moments):
    """Ragged shapes (one side above and one below a tile), two groups, six
    steps with the bases refreshed after steps 2, 4 and 6 (the first from
    the identity, a cold start)."""
    w = _run([(96, 160, 2), (200, 72, 1)], precision, 6, precond_freq=2, soap_moments=moments)
    print("worst", w)


def test_soap_bf16_gradients_and_tiny_sides():
    """bf16 gradients; sides of 1, 7 and 33 (one Jacobi pair block, mostly padding)."""
    _run([(33, 7, 2), (1, 40, 1), (5, 1, 1)], "fp32", 4, grad_dtype="bf16", precond_freq=1)


def test_soap_no_bias_correction_and_every_step_refresh():
    _run([(64, 128, 1)], "fp32", 3, precond_freq=1, bias_correction=0)


@pytest.mark.parametrize("d", [200, 513, 1024])
def test_soap_refresh_recovers_a_known_spectrum(d):
    """A factor with known eigenvectors and eigenvalues spread over 1e-3..1
    (distinct), the identity as the warm start: after one refresh (zero
    gradient, so the factor only decays by soap_beta) Q^T S Q is diagonal
    with S's eigenvalues; a second refresh from that basis keeps it."""
    torch = _torch()
    opt, params = _make([(d, 16, 1)], "fp32", precond_freq=1, soap_beta=0.5)
    rng = np.random.default_rng(d)
    Q0, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.logspace(0, -3, d)
    Lm = (Q0 * lam) @ Q0.T
    opt.state[0]["Sa"][0].copy_(torch.tensor(Lm, dtype=torch.float32))
    zero = torch.zeros(1, d, 16, device="cuda:0")
    for t in (1, 2):
        Lin = opt.state[0]["Sa"][0].double().cpu().numpy()
        opt.step(grads=[zero])
        torch.cuda.synchronize()
        Q = opt.state[0]["Pa"][0].double().cpu().numpy()
        Lout = 0.5 * Lin
        res, orth, eig = S.offdiag_residual(Q, Lout), S.orthogonality(Q), _eig_err(Q, Lout)
        print(f"d={d} refresh {t}: residual {res:.2e} orthogonality {orth:.2e} eigenvalues {eig:.2e}", flush=True)
        assert res < 2e-5 and orth < 2e-5 and eig < 2e-5


@pytest.mark.parametrize("precision", ["fp32", "fp16"])
def test_soap_apply_tile_walk_is_bitwise_one_tile_per_block(precision):
    """The rotation apply run with four tiles per workgroup (the next tile's
    loads in flight during the current products; the form large rounds
    take) gives bitwise the state of one tile per workgroup.  Ragged sides
    (96, 160, 200, 72 and 513) put the walk across the boundary between B
    and V tiles and over partial edge tiles; refreshes after steps 2 and 4,
    the first from the identity."""
    torch = _torch()
    groups = [(96, 160, 2), (200, 72, 1), (513, 40, 1)]
    states = []
    for tiles in (1, 4):
        opt, params = _make(groups, precision, precond_freq=2, jacobi_apply_tiles=tiles)
        for t in range(1, 5):
            grads = [torch.tensor((0.02 * np.random.default_rng([gi, t, 91]).standard_normal((b, m, n))).astype(np.float32),
                                  device="cuda:0") for gi, (m, n, b) in enumerate(groups)]
            opt.step(grads=grads)
        torch.cuda.synchronize()
        states.append([p.clone() for p in params] + [s[k].clone() for s in opt.state for k in sorted(s)])
    for a, b in zip(*states):
        assert torch.equal(a, b)
