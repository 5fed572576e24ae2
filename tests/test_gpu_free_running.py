"""Free-running trajectories of the HIP path beside the fp64 oracle's, as
diagnostics next to the teacher-forced parity tests.

The GPU and the oracle each run the 128 x 256 workload (muP initial
weights, N(0,1) gradients from seed 0) for 20 steps from the same initial
state, each on its own state.  The OKLS factors are updated with the
previous step's roots ("Online KL Shampoo" README, "How it works"), so any
difference in a root feeds into every later factor, and the trajectories
drift apart by more than one step's error; how far is what this reports, per
step, against two oracle runs: the fp64 run of the same damped Newton-Schulz
iteration (the GPU's algorithm in exact arithmetic) and the exact eigh roots
(the method's definition).  Early factors are rank deficient, where the
exact root's gain on the eps-level null space (eps^-1/2) is far from what
the iteration resolves, so the exact-root trajectory is reported only.

Asserted: every state finite, and the weight displacement W_t - W_0 against
the same-iteration oracle's within a bound read off the measured drift with
a margin (the teacher-forced tests carry the per-step tolerances).
"""
import numpy as np
import pytest

from kronecker_factored_second_amd import workloads as WL
from oracle import okls_oracle as O

from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

DRIFT_BOUND = {"fp16": 0.2, "fp32": 0.05}


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_c1_free_running(precision):
    torch = pytest.importorskip("torch")
    w = WL.workload("c1")
    WL.reset_caches()
    opt, params = H.make([(128, 256, 1)], precision=precision)
    W0 = WL.initial_weights(w, 0, 0).astype(np.float32).astype(np.float64)   # the values the GPU holds
    params[0][0].copy_(torch.tensor(W0, device="cuda:0"))
    hp = H.hyper_of(opt)
    rep = H.Report(f"free-c1-{precision}")
    st = {r: O.init_state(W0, hp.eps) for r in ("ns", "exact")}
    worst = 0.0
    for t in range(1, 21):
        G = WL.gradient(w, 0, 0, t)
        opt.step(grads=[H.to_device_grad(G[None], "f32")])
        torch.cuda.synchronize()
        g = H.snapshot(opt, 0, 0)
        assert all(np.all(np.isfinite(x)) for x in (g.W, g.M, g.Sa, g.Sb, g.Pa, g.Pb)), f"t={t}: non-finite state"
        row = dict(t=t)
        for r in ("ns", "exact"):
            st[r] = O.step(st[r], G, hp, t, "okls", root=r).state
            o = st[r]
            row[f"W_{r}"] = O.rel_frob(g.W - W0, o.W - W0)
            row[f"S_a_{r}"] = O.rel_frob(g.Sa, o.Sa)
            row[f"S_b_{r}"] = O.rel_frob(g.Sb, o.Sb)
            row[f"P_a_{r}"] = O.rel_frob(g.Pa, o.Pa)
            row[f"P_b_{r}"] = O.rel_frob(g.Pb, o.Pb)
        rep.add(**row)
        worst = max(worst, row["W_ns"])
        assert row["W_ns"] <= DRIFT_BOUND[precision], row
    print(f"[free-c1-{precision}] worst weight drift against the same iteration {worst:.3e}", flush=True)
