"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare each step against the fp64 oracle started from the GPU's own
previous state (teacher forcing)."""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

from oracle import okls_oracle as O


def _torch():
    import torch
    return torch


def make(groups, precision="fp16", mode="okls", grad_dtype="f32", **cfg):
    """groups: list of (m, n, batch).  Returns (opt, params)."""
    torch = _torch()
    from kronecker_factored_second_amd import okls
    dev = torch.device("cuda:0")
    params = [torch.zeros(b, m, n, device=dev) for (m, n, b) in groups]
    gdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    opt = okls.OKLS(params, mode=mode, precision=precision, grad_dtype=gdt, **cfg)
    return opt, params


def hyper_of(opt, lr=None):
    c = opt.cfg
    return O.Hyper(lr=opt.lr if lr is None else lr, beta1=c.beta1, beta2=c.beta2, eps=c.eps,
                   weight_decay=c.weight_decay, lr_peak=c.lr_peak, nesterov_var_corr=bool(c.nesterov_var_corr),
                   ns_steps=c.ns_steps, ns_floor=float(np.float32(c.ns_floor)), ns_damping=float(np.float32(c.ns_damping)),
                   root_period=int(c.root_period), eps_convex=bool(c.eps_convex), decay_after=bool(c.decay_after),
                   shape_scale=bool(c.shape_scale), ns_classical=bool(c.ns_classical))


def snapshot(opt, gi, idx):
    """fp64 host copy of matrix idx of group gi."""
    s = opt.state[gi]
    f = lambda t: t[idx].detach().double().cpu().numpy()
    return O.MatState(W=f(opt.params[gi]), M=f(s["M"]), Sa=f(s["Sa"]), Sb=f(s["Sb"]), Pa=f(s["Pa"]), Pb=f(s["Pb"]))


def to_device_grad(G: np.ndarray, dtype: str):
    torch = _torch()
    g = torch.tensor(G, device="cuda:0")
    return g.to({"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype])


class Report:
    def __init__(self, name):
        self.name = name
        self.rows = []

    def add(self, **kw):
        self.rows.append(kw)
        msg = " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in kw.items())
        print(f"[{self.name}] {msg}", flush=True)
        sys.stdout.flush()
        path = os.environ.get("OKLS_PARITY_LOG")
        if path:
            with open(path, "a") as f:
                f.write(json.dumps({"case": self.name, **kw}) + "\n")


def compare_step(opt, before, after_idx, G, hp, t, mode, gi, idx):
    """Errors of the GPU result for matrix (gi, idx) against the oracle step
    from `before` (the GPU's state before this step)."""
    ref = O.step(before, G.astype(np.float64), hp, t, mode, root="ns")
    try:
        ex = O.step(before, G.astype(np.float64), hp, t, mode, root="exact")
    except np.linalg.LinAlgError:
        # the GPU's fp32 factor can be indefinite at the eps level (1e-9) where
        # its rank is deficient; the exact root is then undefined (reported NaN)
        ex = None
    after = snapshot(opt, gi, idx)
    m, n = G.shape
    decay = 1.0 - hp.lr * hp.weight_decay * (hp.lr / hp.peak())
    cs = O.c_shape(m, n) if hp.shape_scale else 1.0
    # U read back from the weights, inverting the update form the switches select
    if hp.decay_after:
        U_gpu = (before.W - after.W / decay) / (hp.lr * cs)
    else:
        U_gpu = (decay * before.W - after.W) / (hp.lr * cs)
    return dict(
        S_a=O.rel_frob(after.Sa, ref.state.Sa), S_b=O.rel_frob(after.Sb, ref.state.Sb),
        P_a=O.rel_frob(after.Pa, ref.Pa_ns), P_b=O.rel_frob(after.Pb, ref.Pb_ns),
        P_a_exact=O.rel_frob(after.Pa, ex.state.Pa) if ex else float("nan"),
        P_b_exact=O.rel_frob(after.Pb, ex.state.Pb) if ex else float("nan"),
        M=O.rel_frob(after.M, ref.state.M), U=O.rel_frob(U_gpu, ref.U),
        U_exact=O.rel_frob(U_gpu, ex.U) if ex else float("nan"),
        W=O.rel_frob(after.W, ref.state.W), kappa_a=ref.kappa_a, kappa_b=ref.kappa_b,
        finite=bool(np.isfinite(after.Pa).all() and np.isfinite(after.Pb).all() and np.isfinite(after.W).all()),
    )
