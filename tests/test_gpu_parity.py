"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every step is teacher-forced: the oracle starts from the GPU's own state
before the step and the same gradient.  The preconditioners and the
whitened update are compared with the exact eigh roots of the oracle's new
factors (P = S'^{-1/2}, Shampoo S'^{-1/4}: the "Online KL Shampoo" README,
"How it works"; the Clean paper's eq. (3)), each factor whose condition
number is within its gate (gpu_harness.kappa_gate: 1e3 on the fp16-input
path, 3e2 for sides below 32, 1e4 on the fp32-accurate split path).  A
factor beyond the gate is what ten Newton-Schulz steps in that arithmetic
cannot resolve (the rank-deficient first steps, eps-level null spaces); its
errors are logged, and the whitened update is then asserted against the
oracle's N whitened with the GPU's own roots.  Every root must be finite
and exactly symmetric.

Tolerances (relative Frobenius): factors and preconditioners 2e-2 on the
fp16-input path and 1e-4 on the fp32-accurate path; the whitened update
3e-2; momentum 1e-6.  The measured values go to OKLS_PARITY_LOG when that is
set.
"""
import math

import numpy as np
import pytest

from kronecker_factored_second_amd import workloads as WL
from oracle import okls_oracle as O

from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL = {"fp16": dict(S=2e-2, P=2e-2, U=3e-2, M=1e-6), "fp32": dict(S=1e-4, P=1e-4, U=3e-2, M=1e-6)}


def _assert_step(e, tol, where, precision, ref="exact"):
    """ref 'exact': P and U against the exact roots where the factors are
    within their gates (else U against the GPU's own roots); ref 'ns':
    against the fp64 run of the same iteration (for the classical
    coefficient table, whose own range ends near kappa 1e2)."""
    assert e["finite"], f"non-finite state {where}"
    assert e["P_sym"], f"root not symmetric {where}"
    assert e["M"] < tol["M"], (where, e)
    assert e["S_a"] < tol["S"] and e["S_b"] < tol["S"], (where, e)
    if ref == "ns":
        assert e["P_a_ns"] < tol["P"] and e["P_b_ns"] < tol["P"], (where, e)
        assert e["U_ns"] < tol["U"], (where, e)
        return
    ga, gb, gu = H.gated(e, precision)
    if ga:
        assert e["P_a_exact"] < tol["P"], (where, e)
    if gb:
        assert e["P_b_exact"] < tol["P"], (where, e)
    assert (e["U_exact"] if gu else e["U_whiten"]) < tol["U"], (where, gu, e)


def _run_teacher_forced(name, groups, grad_fn, steps, precision, mode="okls", grad_dtype="f32", check=None,
                        w_init=None, **cfg):
    torch = pytest.importorskip("torch")
    opt, params = H.make(groups, precision=precision, mode=mode, grad_dtype=grad_dtype, **cfg)
    if w_init is not None:
        for gi, (m, n, b) in enumerate(groups):
            for i in range(b):
                params[gi][i].copy_(torch.tensor(w_init(gi, i), device="cuda:0"))
    hp = H.hyper_of(opt)
    rep = H.Report(name)
    tol = TOL[precision]
    worst = {}
    for t in range(1, steps + 1):
        if t > 1:
            # the update is read back from W: zero it after the first step, whose
            # update on rank-deficient factors is large (the root's gain on the
            # directions it does not resolve) and would otherwise swamp a later
            # update in W's fp32 difference
            for p_ in params:
                p_.zero_()
        grads = []
        host = {}
        for gi, (m, n, b) in enumerate(groups):
            gs = [grad_fn(gi, i, t) for i in range(b)]
            host[gi] = gs
            grads.append(H.to_device_grad(np.stack(gs), grad_dtype))
        sel = [(gi, i) for gi, (m, n, b) in enumerate(groups) for i in range(b) if check is None or check(gi, i, t)]
        before = {k: H.snapshot(opt, *k) for k in sel}
        opt.step(grads=grads)
        torch.cuda.synchronize()
        for (gi, i) in sel:
            e = H.compare_step(opt, before[(gi, i)], None, host[gi][i], hp, t, mode, gi, i, precision)
            rep.add(t=t, g=gi, i=i, **e)
            _assert_step(e, tol, f"t={t} group {gi} matrix {i}", precision, "ns" if cfg.get("ns_classical") else "exact")
            ga, gb, gu = H.gated(e, precision)
            for k, on in (("S_a", 1), ("S_b", 1), ("P_a_exact", ga), ("P_b_exact", gb), ("U_exact", gu),
                          ("U_whiten", 1)):
                if on:
                    worst[k] = max(worst.get(k, 0.0), e[k])
    print(f"[{name}] worst {worst}", flush=True)
    return opt


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_c1_all_twenty_steps(precision):
    """128x256 fp32 matrix, N(0,1) gradients from seed 0 for 20 steps."""
    w = WL.workload("c1")
    WL.reset_caches()
    _run_teacher_forced(f"c1-{precision}", [(128, 256, 1)], lambda g, i, t: WL.gradient(w, 0, 0, t), 20, precision,
                        w_init=lambda g, i: WL.initial_weights(w, 0, 0))


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_ragged_shapes_batched(precision):
    """Shapes that are not multiples of the 128 tile, a batch of 3 and a
    matrix smaller than one cast tile."""
    groups = [(200, 72, 3), (130, 300, 1), (33, 40, 2)]

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        r = np.random.default_rng([gi, i, t, 77])
        return (0.02 * r.standard_normal((m, n))).astype(np.float32)

    _run_teacher_forced(f"ragged-{precision}", groups, grad, 3, precision)


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_rank_deficient_tiny_matrices(precision):
    """1 x 7 and 33 x 5 matrices: one factor has rank 1 (or 5) plus the eps
    floor, so its null space lies beyond what any 10-step iteration
    resolves; the resolved directions (the gradient's range) meet the usual
    bounds on S, P and the whitened update."""
    groups = [(1, 7, 1), (33, 5, 2)]

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        return (0.02 * np.random.default_rng([gi, i, t, 78]).standard_normal((m, n))).astype(np.float32)

    _run_teacher_forced(f"rankdef-{precision}", groups, grad, 3, precision)


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_shampoo_mode_small(precision):
    groups = [(96, 160, 2)]

    def grad(gi, i, t):
        return (1e-3 * np.random.default_rng([gi, i, t, 5]).standard_normal((96, 160))).astype(np.float32)

    _run_teacher_forced(f"shampoo-{precision}", groups, grad, 3, precision, mode="shampoo")


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_root_refresh_period(mode, precision):
    """Roots recomputed on steps 1, 4, 7 only (period 3) over ragged shapes:
    on the other steps P stays bitwise what it was, while the factors,
    momentum and the update (whitened with the kept roots) follow the
    oracle's step with the same period.  W is zeroed before every step:
    the first roots of these rank-deficient factors are large, and the
    updates of the steps that keep them grow W far beyond a later step's
    update, which could then not be read back from W's fp32 difference."""
    torch = pytest.importorskip("torch")
    groups = [(96, 160, 2), (130, 72, 1)]
    scale = 0.02 if mode == "okls" else 1e-3

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        return (scale * np.random.default_rng([gi, i, t, 31]).standard_normal((m, n))).astype(np.float32)

    opt, params = H.make(groups, precision=precision, mode=mode, root_period=3)
    hp = H.hyper_of(opt)
    assert hp.root_period == 3
    tol = TOL[precision]
    for t in range(1, 8):
        host = {gi: [grad(gi, i, t) for i in range(b)] for gi, (m, n, b) in enumerate(groups)}
        for p in params:
            p.zero_()
        before = {(gi, i): H.snapshot(opt, gi, i) for gi, (m, n, b) in enumerate(groups) for i in range(b)}
        opt.step(grads=[H.to_device_grad(np.stack(host[gi]), "f32") for gi in range(len(groups))])
        torch.cuda.synchronize()
        for (gi, i), bf in before.items():
            e = H.compare_step(opt, bf, None, host[gi][i], hp, t, mode, gi, i, precision)
            print(f"[period-{mode}-{precision}] t={t} g={gi} i={i} " +
                  " ".join(f"{k}={v:.2e}" for k, v in e.items() if isinstance(v, float)), flush=True)
            _assert_step(e, tol, (t, gi, i), precision)
            after = H.snapshot(opt, gi, i)
            if hp.refresh(t):
                assert not np.array_equal(after.Pa, bf.Pa), (t, gi, i)
            else:
                assert np.array_equal(after.Pa, bf.Pa) and np.array_equal(after.Pb, bf.Pb), (t, gi, i)


def _muon_snapshot(opt, gi, i):
    f = lambda t: t[i].detach().double().cpu().numpy()
    return O.MatState(W=f(opt.params[gi]), M=f(opt.state[gi]["M"]), Sa=None, Sb=None, Pa=None, Pb=None)


@pytest.mark.parametrize("precision,u_tol,gdt", [("fp16", 2e-2, "f32"), ("fp32", 1e-4, "f32"), ("fp16", 2e-2, "f16")])
def test_muon_mode(precision, u_tol, gdt):
    """Muon (polar Newton-Schulz of the momentum, 5 steps) over wide, tall,
    square-ish and tiny shapes (ragged against the tiles), 4 teacher-forced
    steps: M, and the orthogonalised update read back from W (zeroed before
    each step), against the oracle's fp64 iteration."""
    torch = pytest.importorskip("torch")
    groups = [(96, 160, 2), (200, 72, 1), (33, 40, 2), (1, 7, 1)]
    opt, params = H.make(groups, precision=precision, mode="muon", grad_dtype=gdt)
    hp = H.hyper_of(opt)
    assert hp.ns_steps == 5 and abs(hp.ns_floor - 1e-2) < 1e-9
    assert all(set(st) == {"M"} for st in opt.state)          # no factors or roots are allocated
    worst = 0.0
    for t in range(1, 5):
        host = {gi: [(0.02 * np.random.default_rng([gi, i, t, 91]).standard_normal((m, n))).astype(np.float32)
                     for i in range(b)] for gi, (m, n, b) in enumerate(groups)}
        if gdt == "f16":         # values the fp16 gradient holds exactly
            host = {gi: [g.astype(np.float16).astype(np.float32) for g in gs] for gi, gs in host.items()}
        for p in params:
            p.zero_()
        before = {(gi, i): _muon_snapshot(opt, gi, i) for gi, (m, n, b) in enumerate(groups) for i in range(b)}
        opt.step(grads=[H.to_device_grad(np.stack(host[gi]), gdt) for gi in range(len(groups))])
        torch.cuda.synchronize()
        for (gi, i), bf in before.items():
            ref = O.muon_step(bf, host[gi][i].astype(np.float64), hp, t)
            af = _muon_snapshot(opt, gi, i)
            m, n = af.W.shape
            U = -af.W / (hp.lr * O.c_shape(m, n))
            assert np.isfinite(af.W).all()
            e_m, e_u = O.rel_frob(af.M, ref.state.M), O.rel_frob(U, ref.U)
            assert e_m < 1e-6, (t, gi, i, e_m)
            assert e_u < u_tol, (t, gi, i, e_u)
            worst = max(worst, e_u)
    print(f"[muon-{precision}-{gdt}] worst U {worst:.2e}", flush=True)


def test_muon_worked_example_on_gpu():
    """The Shampoo chapter's 2 x 3 gradient through the HIP path in Muon mode
    (split path): the update's singular values are those of the 5-step
    scalar map at sigma / (sum sigma^4)^{1/4}, both within 0.03 of 1 (the
    un-accumulated Shampoo step's 1, 1)."""
    torch = pytest.importorskip("torch")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "shampoo_worked_example.json")))
    G = np.array(g["G"], dtype=np.float32)
    opt, params = H.make([(2, 3, 1)], precision="fp32", mode="muon")
    opt.step(grads=[torch.tensor(G, device="cuda:0")[None]])
    torch.cuda.synchronize()
    hp = H.hyper_of(opt)
    U = -params[0][0].double().cpu().numpy() / (hp.lr * O.c_shape(2, 3))
    sv = np.linalg.svd(U, compute_uv=False)
    coeffs, _ = O.ns_coefficients(hp.ns_floor, hp.ns_steps)
    s = np.array(g["singular_values_G"]) / np.sum(np.array(g["singular_values_G"]) ** 4) ** 0.25
    for a, b in coeffs:
        s = s * (a + b * s * s)
    print(f"[muon-worked-example] sv={sv} expected={s}", flush=True)
    np.testing.assert_allclose(sv, s, atol=2e-3)    # the page prints G's singular values to 3 decimals
    assert np.all(np.abs(sv - 1.0) < 0.03)


@pytest.mark.parametrize("mode,gdt,period,precision", [("okls", "f32", 1, "fp16"), ("shampoo", "f32", 1, "fp16"),
                                                       ("muon", "f32", 1, "fp16"), ("okls", "bf16", 2, "fp16"),
                                                       ("shampoo", "f16", 2, "fp32"), ("muon", "f16", 1, "fp32")])
def test_chunked_steps_are_bitwise_unchunked(mode, gdt, period, precision):
    """chunk_matrices = 1 and 2 (one launch list per chunk, workspace reused)
    give bit-identical states to one chunk: every output element is computed
    by the same kernels in the same order whichever problems share a launch.
    Also with a root period (three steps: refresh, keep, refresh), 16-bit
    gradients and the split path."""
    torch = pytest.importorskip("torch")
    groups = [(96, 160, 2), (130, 72, 1), (33, 40, 2)]
    runs = []
    for chunk in (0, 1, 2):
        opt, params = H.make(groups, precision=precision, mode=mode, grad_dtype=gdt, chunk_matrices=chunk,
                             root_period=period)
        for t in (1, 2, 3):
            grads = [H.to_device_grad((0.02 * np.random.default_rng([gi, t, 17]).standard_normal((b, m, n)))
                                      .astype(np.float32), gdt) for gi, (m, n, b) in enumerate(groups)]
            opt.step(grads=grads)
        torch.cuda.synchronize()
        runs.append([{k: v.cpu().numpy().copy() for k, v in st.items()} | {"W": params[gi].cpu().numpy().copy()}
                     for gi, st in enumerate(opt.state)])
        del opt, params
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            for k in a:
                assert np.array_equal(a[k], b[k]), (mode, gdt, period, precision, k)


@pytest.mark.parametrize("mode,cfg", [("soap", dict(precond_freq=2)), ("nystrom", dict(root_period=2)),
                                      ("nystrom", dict(root_period=1, nys_passes=2))])
def test_chunked_steps_are_bitwise_unchunked_soap_nystrom(mode, cfg):
    """The eigenbasis-Adam and Nystrom modes under chunk_matrices = 1 and 2:
    bit-identical to one chunk over steps that refresh (the bases, the
    low-rank factors) and steps that keep them."""
    torch = pytest.importorskip("torch")
    groups = [(96, 160, 2), (130, 72, 1), (33, 40, 2)]
    runs = []
    for chunk in (0, 1, 2):
        opt, params = H.make(groups, precision="fp32", mode=mode, chunk_matrices=chunk, **cfg)
        for t in (1, 2, 3):
            grads = [H.to_device_grad((0.02 * np.random.default_rng([gi, t, 19]).standard_normal((b, m, n)))
                                      .astype(np.float32), "f32") for gi, (m, n, b) in enumerate(groups)]
            opt.step(grads=grads)
        torch.cuda.synchronize()
        runs.append([{k: v.cpu().numpy().copy() for k, v in st.items()} | {"W": params[gi].cpu().numpy().copy()}
                     for gi, st in enumerate(opt.state)])
        del opt, params
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            for k in a:
                assert np.array_equal(a[k], b[k]), (mode, cfg, k)


@pytest.mark.parametrize("mode", ["okls", "muon"])
def test_step_replays_bitwise_from_a_hip_graph(mode):
    """okls_step captured into a HIP graph (its side-stream fork and join
    included) replays bit-identically to the eager step: three replays, each
    from the same restored state with eager copies in between."""
    torch = pytest.importorskip("torch")
    from kronecker_factored_second_amd import okls
    groups = [(96, 160, 2), (130, 72, 1)]
    grads = [H.to_device_grad((0.02 * np.random.default_rng([gi, 23]).standard_normal((b, m, n))).astype(np.float32), "f32")
             for gi, (m, n, b) in enumerate(groups)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        opt, params = H.make(groups, precision="fp16", mode=mode)
        for _ in range(2):
            opt.step(grads=grads)
        def state():
            return [t for st, p in zip(opt.state, params) for t in (*st.values(), p)]
        saved = [t.clone() for t in state()]
        opt.step(grads=grads)          # eager step t = 3
        torch.cuda.synchronize()
        eager = [t.clone() for t in state()]
        for t, v in zip(state(), saved):
            t.copy_(v)
        tensors = opt._tensors(grads)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            okls.step(opt.handle, tensors, 3, opt.lr, torch.cuda.current_stream().cuda_stream)
        for rep in range(3):
            for t, v in zip(state(), saved):
                t.copy_(v)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(state(), eager):
                assert torch.equal(a, b), (mode, rep)


@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_shampoo_mode_midsize(precision):
    """Factors of 300 and 520 (padded 384 and 768): the second chain's start
    reads the computed square root symmetrised, through its coalesced path in
    whole 64 x 256 blocks and element by element in the edge blocks."""
    groups = [(300, 520, 1)]

    def grad(gi, i, t):
        return (1e-3 * np.random.default_rng([gi, i, t, 6]).standard_normal((300, 520))).astype(np.float32)

    _run_teacher_forced(f"shampoo-mid-{precision}", groups, grad, 2, precision, mode="shampoo")


def test_bf16_gradients_rowscaled():
    """bf16 gradients with per-row log-uniform scales (the transformer-block
    workload's distribution) at a reduced shape spanning several tiles."""
    m, n = 384, 256
    r0 = np.exp(np.random.default_rng(9).uniform(math.log(0.1), math.log(10.0), size=(m, 1)))

    def grad(gi, i, t):
        z = np.random.default_rng([i, t]).standard_normal((m, n))
        return WL.round_to_bf16((0.02 * z * r0).astype(np.float32))

    _run_teacher_forced("bf16-rowscaled", [(m, n, 2)], grad, 3, "fp16", grad_dtype="bf16")


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
def test_f16_gradients_rowscaled(mode):
    """fp16 gradients (the same row-scaled distribution, rounded to fp16 on
    the host so that both sides see identical values, fp16 subnormals
    included) at a ragged shape spanning several tiles."""
    m, n = 330, 270
    r0 = np.exp(np.random.default_rng(10).uniform(math.log(0.1), math.log(10.0), size=(m, 1)))

    def grad(gi, i, t):
        z = np.random.default_rng([i, t, 16]).standard_normal((m, n))
        return (0.02 * z * r0).astype(np.float16).astype(np.float32)

    _run_teacher_forced(f"f16-rowscaled-{mode}", [(m, n, 2)], grad, 3, "fp16", mode=mode, grad_dtype="f16")


def test_shampoo_worked_example_on_gpu():
    """The Shampoo chapter's 2x3 example through the HIP path: the GPU's
    S^{-1/4} factors turn G's singular values (3.377, 1.896) into 1, 1 after
    one accumulation, 0.5 after four and 0.1 after a hundred."""
    torch = pytest.importorskip("torch")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "shampoo_worked_example.json")))
    G = np.array(g["G"], dtype=np.float32)
    opt, params = H.make([(2, 3, 1)], precision="fp32", mode="shampoo")
    gd = torch.tensor(G, device="cuda:0")[None]
    targets = {1: g["singular_values_preconditioned_one_accumulation"],
               4: g["singular_values_after_4_identical_accumulations"],
               100: g["singular_values_after_100_identical_accumulations"]}
    for t in range(1, 101):
        opt.step(grads=[gd])
        if t in targets:
            torch.cuda.synchronize()
            Pa = opt.state[0]["Pa"][0].double().cpu().numpy()
            Pb = opt.state[0]["Pb"][0].double().cpu().numpy()
            sv = np.linalg.svd(Pa @ G.astype(np.float64) @ Pb, compute_uv=False)
            print(f"[worked-example] t={t} sv={sv}", flush=True)
            np.testing.assert_allclose(sv, targets[t], atol=g["printed_precision"])


def test_zero_gradient_is_pure_decay():
    torch = pytest.importorskip("torch")
    opt, params = H.make([(64, 48, 1)], precision="fp16")
    W0 = np.random.default_rng(3).standard_normal((64, 48)).astype(np.float32)
    params[0][0].copy_(torch.tensor(W0, device="cuda:0"))
    opt.step(grads=[torch.zeros(1, 64, 48, device="cuda:0")])
    torch.cuda.synchronize()
    W1 = params[0][0].cpu().numpy().astype(np.float64)
    expect = (1.0 - opt.lr * opt.cfg.weight_decay) * W0.astype(np.float64)
    assert O.rel_frob(W1, expect) < 1e-6
    assert np.all(opt.state[0]["M"].cpu().numpy() == 0.0)


def test_step_is_deterministic():
    torch = pytest.importorskip("torch")
    outs = []
    for _ in range(2):
        opt, params = H.make([(300, 200, 2)], precision="fp16")
        for t in (1, 2):
            g = torch.tensor(np.random.default_rng(t).standard_normal((2, 300, 200)).astype(np.float32), device="cuda:0")
            opt.step(grads=[g])
        torch.cuda.synchronize()
        outs.append([params[0].cpu().clone()] + [opt.state[0][k].cpu().clone() for k in ("M", "Sa", "Sb", "Pa", "Pb")])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_step_is_ordered_on_the_callers_stream():
    """okls_step on a non-default stream: the second Newton-Schulz chain runs on
    the library's side stream, forked from and joined back into the caller's
    stream.  Work the caller queues on its stream right after the step (here
    copies of every state tensor) must see the finished step, and the result
    must equal the default-stream run bit for bit."""
    torch = pytest.importorskip("torch")
    groups = [(256, 384, 2), (512, 128, 1)]

    def run(stream):
        opt, params = H.make(groups, precision="fp16")
        copies = []
        with torch.cuda.stream(stream):
            for t in (1, 2):
                gs = [torch.tensor(np.random.default_rng([t, gi]).standard_normal((b, m, n)).astype(np.float32),
                                   device="cuda:0") for gi, (m, n, b) in enumerate(groups)]
                opt.step(grads=gs)
            for gi in range(len(groups)):
                copies += [params[gi].clone()] + [opt.state[gi][k].clone() for k in ("M", "Sa", "Sb", "Pa", "Pb")]
        torch.cuda.synchronize()
        return [c.cpu() for c in copies]

    ref = run(torch.cuda.default_stream())
    got = run(torch.cuda.Stream())
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mode,switches", [("okls", dict(eps_convex=1, decay_after=1)), ("okls", dict(shape_scale=0)),
                                           ("shampoo", dict(decay_after=1, shape_scale=0)),
                                           ("okls", dict(ns_classical=1)), ("shampoo", dict(ns_classical=1))])
@pytest.mark.parametrize("precision", ["fp16", "fp32"])
def test_reading_switches(mode, switches, precision):
    """The readings kept as switches (R1 convex eps, R6 decay after the
    update, R7 plain update without c_shape, R4's classical coefficient
    table), teacher-forced against the oracle's step with the same switches
    over ragged shapes.  The classical table is checked against the fp64 run
    of its own iteration: ten classical steps reach the exact root only up to
    a condition number of about 1e2."""
    groups = [(96, 160, 2), (130, 72, 1)]
    scale = 0.02 if mode == "okls" else 1e-3

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        return (scale * np.random.default_rng([gi, i, t, 77]).standard_normal((m, n))).astype(np.float32)

    tag = "-".join(f"{k}{v}" for k, v in switches.items())
    _run_teacher_forced(f"switches-{mode}-{tag}-{precision}", groups, grad, 3, precision, mode=mode, **switches)


def test_plain_shampoo_worked_example_in_the_weights():
    """The original Shampoo step through the HIP path (no momentum, decay or
    c_shape; lr 1; split path): the weight steps W_{t-1} - W_t
    on the worked example's repeated G have the page's singular values 1, 1
    after one accumulation, 0.5 after four and 0.1 after a hundred."""
    torch = pytest.importorskip("torch")
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "shampoo_worked_example.json")))
    G = np.array(g["G"], dtype=np.float32)
    opt, params = H.make([(2, 3, 1)], precision="fp32", mode="shampoo", beta1=0.0,
                         nesterov_var_corr=0, weight_decay=0.0, shape_scale=0)
    opt.lr = 1.0
    gd = torch.tensor(G, device="cuda:0")[None]
    want = {1: g["singular_values_preconditioned_one_accumulation"],
            4: g["singular_values_after_4_identical_accumulations"],
            100: g["singular_values_after_100_identical_accumulations"]}
    for t in range(1, 101):
        W_prev = params[0][0].double().cpu().numpy()
        opt.step(grads=[gd])
        if t in want:
            torch.cuda.synchronize()
            sv = np.linalg.svd(W_prev - params[0][0].double().cpu().numpy(), compute_uv=False)
            print(f"[plain-shampoo] t={t} singular values {sv}", flush=True)
            np.testing.assert_allclose(sv, want[t], atol=g["printed_precision"])


def test_single_chain_plan():
    """A chunk whose single-chain Newton-Schulz launch is exactly one full
    round of 256 tiles (128 matrices of 256 x 256) runs one chain, with no
    side stream: every 16th matrix teacher-forced for two steps."""
    groups = [(256, 256, 128)]

    def grad(gi, i, t):
        return (0.02 * np.random.default_rng([i, t, 256]).standard_normal((256, 256))).astype(np.float32)

    opt = _run_teacher_forced("single-chain", groups, grad, 2, "fp16", check=lambda gi, i, t: i % 16 == 0)
    from kronecker_factored_second_amd import okls
    assert okls.workspace_size(opt.cfg, opt.groups) > 0


def test_maximum_group_count():
    """Sixteen groups, the most one handle takes, of distinct ragged shapes
    (tall, wide, square, vectors; batches 1 and 2) in one step: the
    per-group pointer table at capacity, teacher-forced for two steps."""
    rng = np.random.default_rng(1616)
    groups = []
    while len(groups) < 16:
        m, n = (int(x) for x in rng.integers(1, 200, size=2))
        if all((m, n) != (a, b) for a, b, _ in groups):
            groups.append((m, n, int(rng.integers(1, 3))))

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        return (0.02 * np.random.default_rng([gi, i, t, 161]).standard_normal((m, n))).astype(np.float32)

    _run_teacher_forced("sixteen-groups", groups, grad, 2, "fp16")


def test_many_small_matrices():
    """Thousands of small matrices in one step (2048 of 8 x 8 and 1024 of
    12 x 20): thousands of statistics, cast and GEMM problems per launch,
    each padded to one 128 tile; every matrix teacher-forced for two steps."""
    groups = [(8, 8, 2048), (12, 20, 1024)]

    def grad(gi, i, t):
        m, n, _ = groups[gi]
        return (0.02 * np.random.default_rng([gi, i, t, 2048]).standard_normal((m, n))).astype(np.float32)

    _run_teacher_forced("many-small", groups, grad, 2, "fp16")


@pytest.mark.parametrize("mode,period", [("okls", 2), ("shampoo", 1), ("muon", 1)])
def test_checkpoint_resume_is_bitwise(tmp_path, mode, period):
    """state_dict() after two steps, saved with torch.save and read back with
    weights_only=True into a fresh optimizer (new handle and workspace), then
    two more steps: bit-identical to four uninterrupted steps.  With a root
    period of 2 the first step after the resume keeps the roots, so the
    library carries nothing between steps beyond the caller's state and t."""
    torch = pytest.importorskip("torch")
    groups = [(96, 160, 2), (33, 40, 1)]

    def grads(t):
        return [H.to_device_grad((0.02 * np.random.default_rng([gi, t, 29]).standard_normal((b, m, n)))
                                 .astype(np.float32), "f32") for gi, (m, n, b) in enumerate(groups)]

    def fresh():
        opt, params = H.make(groups, precision="fp16", mode=mode, root_period=period)
        for gi, p in enumerate(params):
            p.copy_(0.01 * torch.ones_like(p) * (gi + 1))
        return opt, params

    ref, ref_p = fresh()
    for t in range(1, 5):
        ref.step(grads=grads(t))
    a, a_p = fresh()
    for t in (1, 2):
        a.step(grads=grads(t))
    torch.save({"opt": a.state_dict(), "params": [p.detach().clone() for p in a_p]}, tmp_path / "ckpt.pt")
    del a, a_p
    ck = torch.load(tmp_path / "ckpt.pt", weights_only=True)
    b, b_p = fresh()
    b.load_state_dict(ck["opt"])
    for p, q in zip(b_p, ck["params"]):
        p.copy_(q)
    assert b.t == 2
    for t in (3, 4):
        b.step(grads=grads(t))
    torch.cuda.synchronize()
    for gi in range(len(groups)):
        assert torch.equal(ref_p[gi], b_p[gi]), (mode, gi, "W")
        for k in ref.state[gi]:
            assert torch.equal(ref.state[gi][k], b.state[gi][k]), (mode, gi, k)


def test_step_argument_errors_launch_nothing():
    """okls_step's host checks through the C ABI on a live handle: t < 1, a
    non-finite or negative lr, missing tensors, a null or misaligned G each
    return OKLS_ERR_INVALID_ARG before any launch (the state stays
    bit-identical), and a valid step still runs afterwards."""
    import ctypes
    torch = pytest.importorskip("torch")
    from kronecker_factored_second_amd import okls
    opt, params = H.make([(64, 48, 1)], precision="fp16")
    lib = okls.load()
    g = torch.zeros(1, 64, 48, device="cuda:0")
    before = {k: v.clone() for k, v in opt.state[0].items()} | {"W": params[0].clone()}
    good = opt._tensors([g])
    s = ctypes.c_void_p(opt.stream)
    assert lib.okls_step(opt.handle, good, 0, ctypes.c_float(0.1), s) == -1
    assert lib.okls_step(opt.handle, good, 1, ctypes.c_float(float("nan")), s) == -1
    assert lib.okls_step(opt.handle, good, 1, ctypes.c_float(-0.1), s) == -1
    assert lib.okls_step(opt.handle, None, 1, ctypes.c_float(0.1), s) == -1
    no_g = opt._tensors([g])
    no_g[0].G = None
    assert lib.okls_step(opt.handle, no_g, 1, ctypes.c_float(0.1), s) == -1
    odd = opt._tensors([g])
    odd[0].G = g.data_ptr() + 2                   # fp32 G must be 4-byte aligned
    assert lib.okls_step(opt.handle, odd, 1, ctypes.c_float(0.1), s) == -1
    no_s = opt._tensors([g])
    no_s[0].Sa = None
    assert lib.okls_step(opt.handle, no_s, 1, ctypes.c_float(0.1), s) == -1
    assert lib.okls_check_finite(opt.handle, None, s) == -1
    assert lib.okls_profile_read(opt.handle, None) == -1
    torch.cuda.synchronize()
    after = {k: v for k, v in opt.state[0].items()} | {"W": params[0]}
    for k in before:
        assert torch.equal(before[k], after[k]), k
    assert lib.okls_step(opt.handle, good, 1, ctypes.c_float(0.1), s) == 0
    torch.cuda.synchronize()
    assert not torch.equal(before["Pa"], opt.state[0]["Pa"])


def test_step_reads_p_grad():
    """step() without grads reads each parameter's .grad (2-D parameters, as a
    model holds them): bit-identical to passing the same tensors explicitly;
    a parameter without a gradient is refused."""
    torch = pytest.importorskip("torch")
    from kronecker_factored_second_amd import okls
    shapes = [(96, 160), (40, 33)]
    runs = []
    for explicit in (False, True):
        params = [torch.zeros(m, n, device="cuda:0") for m, n in shapes]
        opt = okls.OKLS(params, precision="fp16")
        for t in (1, 2):
            gs = [torch.tensor((0.02 * np.random.default_rng([i, t]).standard_normal(s_)).astype(np.float32),
                               device="cuda:0") for i, s_ in enumerate(shapes)]
            if explicit:
                opt.step(grads=gs)
            else:
                for p_, g in zip(params, gs):
                    p_.grad = g
                opt.step()
                opt.zero_grad()
        torch.cuda.synchronize()
        runs.append([p_.clone() for p_ in params] + [v.clone() for st in opt.state for v in st.values()])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    with pytest.raises(ValueError):
        opt.step()                      # zero_grad() left no gradients


def test_step_refuses_mismatched_gradients():
    """The wrapper refuses a gradient whose dtype, shape or presence differs
    from what the handle was built for (the library would misread it, or read
    past its end), before anything is launched: the step counter and the
    state are untouched."""
    torch = pytest.importorskip("torch")
    opt, params = H.make([(64, 48, 2)], precision="fp16", grad_dtype="bf16")
    good = torch.zeros(2, 64, 48, device="cuda:0", dtype=torch.bfloat16)
    M0 = opt.state[0]["M"].clone()
    for bad in (good.float(), good.half(), good[:1], torch.zeros(2, 48, 64, device="cuda:0", dtype=torch.bfloat16),
                good.cpu(), None):
        with pytest.raises(ValueError):
            opt.step(grads=[bad])
    with pytest.raises(ValueError):
        opt.step(grads=[good, good])
    assert opt.t == 0 and torch.equal(opt.state[0]["M"], M0)
    opt.step(grads=[good])
    torch.cuda.synchronize()
    assert opt.t == 1


@pytest.mark.parametrize("mode", ["okls", "shampoo"])
def test_factor_gemm_matches_fp64_on_exact_fp16_inputs(mode):
    """The GEMM on inputs the fp16 cast represents exactly: G holds
    fp16-representable values and the cast's scale is a power of two, so at
    t = 1 (P = I) the factor update multiplies exactly G.  S_1 minus its eps
    terms then equals c1 G G^T (c1 = (1 - beta2)/n or 1) to fp32 accumulation
    accuracy, over a ragged 300 x 520 matrix (K = 520 and 300)."""
    torch = pytest.importorskip("torch")
    m, n = 300, 520
    G = (np.random.default_rng(37).standard_normal((m, n)).astype(np.float16).astype(np.float64)) * 0.125
    opt, params = H.make([(m, n, 1)], precision="fp16", mode=mode)
    hp = H.hyper_of(opt)
    opt.step(grads=[torch.tensor(G.astype(np.float32), device="cuda:0")[None]])
    torch.cuda.synchronize()
    okls_mode = mode == "okls"
    c0 = hp.beta2 if okls_mode else 1.0
    for key, gram, den in (("Sa", G @ G.T, n), ("Sb", G.T @ G, m)):
        c1 = (1.0 - hp.beta2) / den if okls_mode else 1.0
        d = gram.shape[0]
        want = c1 * gram + (c0 * hp.eps + hp.eps) * np.eye(d)
        got = opt.state[0][key][0].double().cpu().numpy()
        err = O.rel_frob(got, want)
        print(f"[exact-gemm-{mode}] {key} rel err {err:.2e}", flush=True)
        assert err < 1e-5, (key, err)


def test_factors_are_exactly_symmetric():
    """The factor update computes the upper triangle and mirrors it, so S_a
    and S_b are bitwise symmetric after every step (both modes, ragged
    shapes, three steps)."""
    torch = pytest.importorskip("torch")
    groups = [(200, 72, 1), (130, 300, 1), (33, 40, 2)]
    for mode in ("okls", "shampoo"):
        opt, params = H.make(groups, precision="fp16", mode=mode)
        for t in (1, 2, 3):
            opt.step(grads=[H.to_device_grad((0.02 * np.random.default_rng([gi, t, 53]).standard_normal((b, m, n)))
                                             .astype(np.float32), "f32") for gi, (m, n, b) in enumerate(groups)])
            torch.cuda.synchronize()
            for st in opt.state:
                for k in ("Sa", "Sb"):
                    assert torch.equal(st[k], st[k].transpose(1, 2)), (mode, t, k)


@pytest.mark.parametrize("precision,tol", [("fp16", 2e-2), ("fp32", 1e-4)])
def test_diagonal_factor_follows_the_scalar_recurrence(precision, tol):
    """A diagonal factor with distinct eigenvalues (log-uniform over kappa 1e3)
    and a zero gradient: every Newton-Schulz iterate stays diagonal, so P is
    exactly diagonal and each entry is the oracle's scalar recurrence
    (ns_spectral) at beta2 lambda + eps, over d = 300 (ragged against the
    tiles)."""
    torch = pytest.importorskip("torch")
    d, n = 300, 40
    opt, params = H.make([(d, n, 1)], precision=precision)
    hp = H.hyper_of(opt)
    lam = np.exp(np.random.default_rng(19).uniform(np.log(1e-3), 0.0, d)) * 1e-4
    lam32 = lam.astype(np.float32)
    opt.state[0]["Sa"][0].copy_(torch.diag(torch.tensor(lam32)))
    opt.step(grads=[torch.zeros(1, d, n, device="cuda:0")])
    torch.cuda.synchronize()
    P = opt.state[0]["Pa"][0].double().cpu().numpy()
    off = P - np.diag(np.diag(P))
    assert np.count_nonzero(off) == 0
    lam1 = hp.beta2 * lam32.astype(np.float64) + hp.eps
    want = O.ns_spectral(lam1, O.ns_coefficients(hp.ns_floor, hp.ns_steps)[0], hp.ns_damping, 2)
    err = O.rel_frob(np.diag(P), want)
    print(f"[diagonal-{precision}] P vs scalar recurrence {err:.2e}", flush=True)
    assert err < tol


def test_only_the_upper_triangle_of_s_is_read():
    """S must be symmetric on entry and only its upper triangle is read: a
    factor whose lower triangle holds junk gives bit-identically the step of
    the factor with the upper triangle mirrored (both modes)."""
    torch = pytest.importorskip("torch")
    for mode in ("okls", "shampoo"):
        outs = []
        for junk in (False, True):
            opt, params = H.make([(96, 160, 1)], precision="fp16", mode=mode)
            rng = np.random.default_rng(5)
            A = rng.standard_normal((96, 96))
            S = 1e-4 * (A @ A.T / 96 + np.eye(96))
            if junk:
                S = np.triu(S) + np.tril(np.random.default_rng(6).standard_normal((96, 96)), -1)
            opt.state[0]["Sa"][0].copy_(torch.tensor(S, dtype=torch.float32))
            G = 0.02 * np.random.default_rng(7).standard_normal((1, 96, 160))
            g = torch.tensor(G.astype(np.float32), device="cuda:0")
            opt.step(grads=[g])
            torch.cuda.synchronize()
            outs.append({k: v.clone() for k, v in opt.state[0].items()} | {"W": params[0].clone()})
        for k in outs[0]:
            assert torch.equal(outs[0][k], outs[1][k]), (mode, k)


def test_nan_gradient_is_detected():
    """A NaN in the gradient reaches the momentum and the update, and
    okls_check_finite reports it (OKLS_ERR_NONFINITE through the binding)."""
    torch = pytest.importorskip("torch")
    opt, params = H.make([(64, 48, 1)], precision="fp16")
    g = torch.zeros(1, 64, 48, device="cuda:0")
    g[0, 5, 7] = float("nan")
    opt.step(grads=[g])
    assert not opt.check_finite()
    assert torch.isnan(opt.state[0]["M"][0, 5, 7])


def test_check_finite_flags_nan():
    torch = pytest.importorskip("torch")
    opt, params = H.make([(64, 64, 1)], precision="fp16")
    assert opt.check_finite()
    opt.state[0]["Sa"][0, 3, 3] = float("nan")
    assert not opt.check_finite()


@pytest.mark.parametrize("precision,tol", [("fp32", 1e-4), ("fp16", 2e-2)])
def test_well_conditioned_state_matches_exact_root(precision, tol):
    """From a factor state with condition number 100 (set through the state
    tensors) and a small gradient, the new factors stay well conditioned and
    the GPU's Newton-Schulz root matches the exact eigh root of the oracle's
    factor over the whole matrix, in the shipped configuration of each path
    (the iteration converges inside its design interval)."""
    torch = pytest.importorskip("torch")
    m, n = 192, 320
    rng = np.random.default_rng(21)

    def spd(d, kappa):
        Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
        lam = np.logspace(0, -np.log10(kappa), d) * 1e-3
        return (Q * lam) @ Q.T

    opt, params = H.make([(m, n, 1)], precision=precision)
    Sa, Sb = spd(m, 100.0), spd(n, 100.0)
    Pa, _ = O.inv_root_exact(Sa, 2)
    Pb, _ = O.inv_root_exact(Sb, 2)
    st = opt.state[0]
    for k, v in (("Sa", Sa), ("Sb", Sb), ("Pa", Pa), ("Pb", Pb)):
        st[k][0].copy_(torch.tensor(v, dtype=torch.float32, device="cuda:0"))
    params[0][0].copy_(torch.tensor(rng.standard_normal((m, n)) * 0.01, dtype=torch.float32, device="cuda:0"))
    hp = H.hyper_of(opt)
    rep = H.Report(f"wellcond-{precision}")
    for t in (1, 2):
        G = (1e-3 * rng.standard_normal((m, n))).astype(np.float32)
        before = H.snapshot(opt, 0, 0)
        opt.step(grads=[torch.tensor(G, device="cuda:0")[None]])
        torch.cuda.synchronize()
        e = H.compare_step(opt, before, None, G, hp, t, "okls", 0, 0, precision)
        rep.add(t=t, **e)
        assert e["kappa_a"] < 1e3 and e["kappa_b"] < 1e3
        assert e["P_a_exact"] < tol and e["P_b_exact"] < tol, e
        assert e["U_exact"] < max(tol, 1e-3), e


@pytest.mark.parametrize("mode,cfg", [("okls", {}), ("soap", dict(precond_freq=2)), ("nystrom", dict(root_period=2))])
def test_misaligned_weights_take_the_scalar_path(mode, cfg):
    """W as a view one float into its buffer (4-byte aligned, not 16): the
    fp32 epilogues use their element-wise path and give bit-identically the
    results of an aligned W over three steps (factor update, weight update;
    SOAP's and Nystrom's weight updates and refreshes)."""
    torch = pytest.importorskip("torch")
    from kronecker_factored_second_amd import okls
    m, n = 96, 160
    W0 = torch.tensor(np.random.default_rng(71).standard_normal((1, m, n)).astype(np.float32) * 0.01, device="cuda:0")
    buf = torch.zeros(1 + m * n, device="cuda:0")
    Wodd = buf[1:].view(1, m, n)
    assert Wodd.data_ptr() % 16 == 4
    runs = []
    for W in (W0.clone(), Wodd):
        W.copy_(W0)
        opt = okls.OKLS([W], precision="fp16", mode=mode, **cfg)
        for t in (1, 2, 3):
            g = torch.tensor((0.02 * np.random.default_rng([t, 72]).standard_normal((1, m, n))).astype(np.float32),
                             device="cuda:0")
            opt.step(grads=[g])
        torch.cuda.synchronize()
        runs.append([W.clone()] + [opt.state[0][k].clone() for k in sorted(opt.state[0])])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_refused_step_and_mismatched_checkpoint_change_nothing():
    """A step the library refuses (a non-finite learning rate) does not
    advance the step counter; load_state_dict refuses a checkpoint with the
    wrong parameter count, keys or shapes before copying anything."""
    torch = pytest.importorskip("torch")
    from kronecker_factored_second_amd import okls
    opt, params = H.make([(64, 48, 1), (32, 40, 2)], precision="fp16")
    grads = [torch.zeros(1, 64, 48, device="cuda:0"), torch.zeros(2, 32, 40, device="cuda:0")]
    with pytest.raises(okls.OKLSError):
        opt.step(grads=grads, lr=float("nan"))
    assert opt.t == 0 and opt.lr == pytest.approx(0.09434)
    opt.step(grads=grads, lr=0.05)
    assert opt.t == 1
    sd = opt.state_dict()
    before = [{k: v.clone() for k, v in s.items()} for s in opt.state]
    bad_count = dict(sd, state=sd["state"][:1])
    bad_keys = dict(sd, state=[{k: v for k, v in s.items() if k != "Pa"} for s in sd["state"]])
    bad_shape = dict(sd, state=[dict(s, M=s["M"][:, :-1]) for s in sd["state"]])
    for bad in (bad_count, bad_keys, bad_shape):
        opt.t = 7
        with pytest.raises(ValueError):
            opt.load_state_dict(bad)
        assert opt.t == 7
        for s, b in zip(opt.state, before):
            for k in s:
                assert torch.equal(s[k], b[k])
    opt.load_state_dict(sd)
    assert opt.t == 1
