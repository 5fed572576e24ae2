"""Thin Python binding of libokls.so (the C ABI declared in include/okls.h).

Argument marshalling only: every step of the optimizer runs in the HIP
library.  PyTorch supplies device memory and the current stream.  The
functions keep the C names; `OKLS` is a convenience wrapper that owns the
state tensors and the workspace of a list of matrix parameters.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libokls.so")

OKLS_OK = 0
STATUS = {0: "OKLS_OK", -1: "OKLS_ERR_INVALID_ARG", -2: "OKLS_ERR_SHAPE", -3: "OKLS_ERR_DTYPE",
          -4: "OKLS_ERR_WORKSPACE", -5: "OKLS_ERR_HIP", -6: "OKLS_ERR_NONFINITE", -7: "OKLS_ERR_UNSUPPORTED"}
OKLS_F32, OKLS_BF16, OKLS_F16 = 0, 1, 2
MODE = {"okls": 0, "shampoo": 1, "muon": 2, "soap": 3, "nystrom": 4}
# the Muon setting of the polar iteration: 5 steps (Clean, Table 6) on [1e-2, 1]
MUON_DEFAULTS = dict(ns_steps=5, ns_floor=1e-2)
# optimizer hyperparameters per mode: the README's "Hyperparameters" table, and
# SOAP's from the Clean paper's Tables 4 and 6
HYPER_DEFAULTS = {"okls": dict(lr=0.09434, beta1=0.9684, beta2=0.9482, eps=1e-9, weight_decay=0.0303),
                  "soap": dict(lr=2.8e-3, beta1=0.95, beta2=0.95, eps=1e-8, weight_decay=0.1)}
EXPORTED = ("okls_default_config", "okls_workspace_size", "okls_init", "okls_init_state", "okls_step",
            "okls_check_finite", "okls_ns_coefficients", "okls_profile_enable", "okls_profile_read",
            "okls_destroy", "okls_status_string", "okls_plan_query", "okls_init_static", "okls_ns_residuals")
STATIC_SCRATCH_BYTES = 128 << 20
PROFILE_CATEGORIES = ("ns_gemm", "factor_gemm", "whiten_gemm", "stats", "cast", "eigensolver")


class Config(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("ns_steps", ctypes.c_int32), ("ns_split_steps", ctypes.c_int32),
                ("factor_split", ctypes.c_int32), ("nesterov_var_corr", ctypes.c_int32),
                ("chunk_matrices", ctypes.c_int32), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("lr_peak", ctypes.c_float),
                ("ns_floor", ctypes.c_float), ("ns_damping", ctypes.c_float), ("root_period", ctypes.c_int32),
                ("eps_convex", ctypes.c_int32), ("decay_after", ctypes.c_int32), ("shape_scale", ctypes.c_int32),
                ("ns_classical", ctypes.c_int32), ("whiten_split", ctypes.c_int32),
                ("soap_beta", ctypes.c_float), ("precond_freq", ctypes.c_int32), ("soap_moments", ctypes.c_int32),
                ("bias_correction", ctypes.c_int32), ("jacobi_sweeps", ctypes.c_int32), ("jacobi_tol", ctypes.c_float),
                ("nys_rank", ctypes.c_int32), ("nys_oversample", ctypes.c_int32), ("nys_passes", ctypes.c_int32),
                ("jacobi_apply_tiles", ctypes.c_int32)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("g_dtype", ctypes.c_int32)]


class GroupTensors(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("G", ctypes.c_void_p), ("M", ctypes.c_void_p), ("Sa", ctypes.c_void_p),
                ("Sb", ctypes.c_void_p), ("Pa", ctypes.c_void_p), ("Pb", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("PsiA", ctypes.c_void_p), ("PsiB", ctypes.c_void_p)]


class ProfileStats(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 6), ("busy_ms", ctypes.c_double * 6), ("flops", ctypes.c_double * 6),
                ("bytes", ctypes.c_double * 6),
                ("launches", ctypes.c_int64 * 6), ("steps", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("chunks", ctypes.c_int32), ("launches", ctypes.c_int32), ("launches_stale", ctypes.c_int32),
                ("ns_chains", ctypes.c_int32), ("flops", ctypes.c_double * 6), ("bytes", ctypes.c_double * 6)]


class OKLSError(RuntimeError):
    def __init__(self, call, status):
        self.status = status
        super().__init__(f"{call} failed: {STATUS.get(status, status)}")


_lib = None


def load(path: str = LIB_PATH):
    """Loads libokls.so; raises if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.okls_default_config.argtypes = [ctypes.POINTER(Config)]
    lib.okls_default_config.restype = None
    lib.okls_workspace_size.argtypes = [ctypes.POINTER(Config), ctypes.c_int, ctypes.POINTER(GroupDesc)]
    lib.okls_workspace_size.restype = sz
    lib.okls_init.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(Config), ctypes.c_int,
                              ctypes.POINTER(GroupDesc), vp, sz, vp]
    lib.okls_init.restype = ctypes.c_int
    lib.okls_init_static.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(Config), ctypes.c_int,
                                     ctypes.POINTER(GroupDesc), vp]
    lib.okls_init_static.restype = ctypes.c_int
    lib.okls_init_state.argtypes = [vp, ctypes.POINTER(GroupTensors), vp]
    lib.okls_init_state.restype = ctypes.c_int
    lib.okls_step.argtypes = [vp, ctypes.POINTER(GroupTensors), i64, f32, vp]
    lib.okls_step.restype = ctypes.c_int
    lib.okls_check_finite.argtypes = [vp, ctypes.POINTER(GroupTensors), vp]
    lib.okls_check_finite.restype = ctypes.c_int
    lib.okls_ns_residuals.argtypes = [vp, ctypes.POINTER(ctypes.c_double), i64, vp]
    lib.okls_ns_residuals.restype = ctypes.c_int
    lib.okls_ns_coefficients.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.okls_ns_coefficients.restype = ctypes.c_int
    lib.okls_profile_enable.argtypes = [vp, ctypes.c_int]
    lib.okls_profile_enable.restype = ctypes.c_int
    lib.okls_profile_read.argtypes = [vp, ctypes.POINTER(ProfileStats)]
    lib.okls_profile_read.restype = ctypes.c_int
    lib.okls_destroy.argtypes = [vp]
    lib.okls_destroy.restype = ctypes.c_int
    lib.okls_plan_query.argtypes = [ctypes.POINTER(Config), ctypes.c_int, ctypes.POINTER(GroupDesc),
                                    ctypes.POINTER(PlanInfo)]
    lib.okls_plan_query.restype = ctypes.c_int
    lib.okls_status_string.argtypes = [ctypes.c_int]
    lib.okls_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(call, st):
    if st != OKLS_OK:
        raise OKLSError(call, st)


# --------------------------------------------------------------------------
# One-to-one wrappers of the C entry points
# --------------------------------------------------------------------------
def default_config(**overrides) -> Config:
    c = Config()
    load().okls_default_config(ctypes.byref(c))
    for k, v in overrides.items():
        if k == "mode" and isinstance(v, str):
            v = MODE[v]
        setattr(c, k, v)
    return c


def precision_config(precision: str = "fp16", **overrides) -> Config:
    """'fp16': the Newton-Schulz and factor GEMMs with plain fp16 inputs (the
    pages' path), the whitening products split-fp16 (whiten_split).
    'fp32': every GEMM split-fp16 (hi*hi + hi*lo + lo*hi), fp32-accurate.
    Each takes the coefficient table's floor matched to its arithmetic.
    (SOAP mode follows factor_split alone: every product split with 'fp32'.)"""
    if precision == "fp16":
        base = dict(ns_split_steps=0, factor_split=0, whiten_split=1, ns_floor=3e-2, ns_damping=0.0)
    elif precision == "fp32":
        base = dict(ns_split_steps=-1, factor_split=1, whiten_split=1, ns_floor=1e-3, ns_damping=0.0)
    else:
        raise ValueError(precision)
    base.update(overrides)
    c = default_config(**{k: v for k, v in base.items() if k != "ns_split_steps"})
    c.ns_split_steps = c.ns_steps if base["ns_split_steps"] == -1 else base["ns_split_steps"]
    return c


def _groups_array(groups):
    arr = (GroupDesc * len(groups))()
    for i, (batch, m, n, gdt) in enumerate(groups):
        arr[i] = GroupDesc(batch, m, n, gdt)
    return arr


def workspace_size(cfg: Config, groups) -> int:
    """groups: list of (batch, m, n, g_dtype)."""
    return int(load().okls_workspace_size(ctypes.byref(cfg), len(groups), _groups_array(groups)))


def plan_query(cfg: Config, groups) -> dict:
    """What a step of these groups runs (host only): chunks, kernel launches of
    a refresh / stale step, concurrent Newton-Schulz chains, and the refresh
    step's algorithmic FLOPs and bytes per profile category."""
    info = PlanInfo()
    st = load().okls_plan_query(ctypes.byref(cfg), len(groups), _groups_array(groups), ctypes.byref(info))
    if st != 0:
        raise OKLSError("okls_plan_query", st)
    return {"chunks": info.chunks, "launches": info.launches, "launches_stale": info.launches_stale,
            "ns_chains": info.ns_chains,
            "flops": dict(zip(PROFILE_CATEGORIES, info.flops)), "bytes": dict(zip(PROFILE_CATEGORIES, info.bytes))}


def ns_coefficients(cfg: Config):
    a = (ctypes.c_double * 32)()
    b = (ctypes.c_double * 32)()
    k = load().okls_ns_coefficients(ctypes.byref(cfg), a, b, 32)
    if k < 0:
        raise OKLSError("okls_ns_coefficients", -1)
    return list(a[:k]), list(b[:k])


def fit_chunk(cfg: Config, groups, limit: int):
    """Largest chunk_matrices whose workspace is at most `limit` bytes, and
    that workspace size (bisection; the size grows with the chunk)."""
    total = sum(g[0] for g in groups)
    saved = cfg.chunk_matrices
    try:
        lo, hi, best = 1, total, None
        while lo <= hi:
            mid = (lo + hi) // 2
            cfg.chunk_matrices = mid
            ws = workspace_size(cfg, groups)
            if ws != 0 and ws <= limit:
                best, lo = (mid, ws), mid + 1
            else:
                hi = mid - 1
    finally:
        cfg.chunk_matrices = saved
    if best is None:
        raise MemoryError(f"one matrix needs more workspace than the limit of {limit} bytes")
    return best


def status_string(st: int) -> str:
    return load().okls_status_string(st).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def tensors_array(per_group):
    """per_group: list of dicts with torch tensors W, G, M, Sa, Sb, Pa, Pb (and V in SOAP mode,
    PsiA and PsiB in Nystrom mode)."""
    arr = (GroupTensors * len(per_group))()
    for i, d in enumerate(per_group):
        arr[i] = GroupTensors(*[(d[k].data_ptr() if d.get(k) is not None else None)
                                for k in ("W", "G", "M", "Sa", "Sb", "Pa", "Pb", "V", "PsiA", "PsiB")])
    return arr


def init(cfg: Config, groups, workspace, stream) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    st = load().okls_init(ctypes.byref(h), ctypes.byref(cfg), len(groups), _groups_array(groups),
                          ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                          ctypes.c_void_p(stream))
    _check("okls_init", st)
    return h


def init_static(cfg: Config, groups, stream) -> ctypes.c_void_p:
    """okls_init_static: a handle whose workspace is the library's static
    device scratch (nothing is allocated on the device)."""
    h = ctypes.c_void_p()
    st = load().okls_init_static(ctypes.byref(h), ctypes.byref(cfg), len(groups), _groups_array(groups),
                                 ctypes.c_void_p(stream))
    _check("okls_init_static", st)
    return h


def init_state(h, tensors, stream):
    _check("okls_init_state", load().okls_init_state(h, tensors, ctypes.c_void_p(stream)))


def step(h, tensors, t: int, lr: float, stream):
    _check("okls_step", load().okls_step(h, tensors, int(t), float(lr), ctypes.c_void_p(stream)))


def check_finite(h, tensors, stream) -> bool:
    st = load().okls_check_finite(h, tensors, ctypes.c_void_p(stream))
    if st == -6:
        return False
    _check("okls_check_finite", st)
    return True


def ns_residuals(h, n_mats: int, stream):
    """||Z_{K-1} Y_{K-1} - I||_F per (matrix, side, chain): a list of
    n_mats entries [[a0, a1], [b0, b1]] (NaN where not computed)."""
    buf = (ctypes.c_double * (4 * n_mats))()
    _check("okls_ns_residuals", load().okls_ns_residuals(h, buf, 4 * n_mats, ctypes.c_void_p(stream)))
    return [[[buf[(i * 2 + s) * 2 + c] for c in range(2)] for s in range(2)] for i in range(n_mats)]


def profile_enable(h, enable: bool):
    _check("okls_profile_enable", load().okls_profile_enable(h, 1 if enable else 0))


def profile_read(h) -> dict:
    st = ProfileStats()
    _check("okls_profile_read", load().okls_profile_read(h, ctypes.byref(st)))
    return {name: {"ms": st.ms[i], "busy_ms": st.busy_ms[i], "flops": st.flops[i], "bytes": st.bytes[i],
                   "launches": int(st.launches[i])}
            for i, name in enumerate(PROFILE_CATEGORIES)} | {"steps": int(st.steps)}


def destroy(h):
    _check("okls_destroy", load().okls_destroy(h))


# --------------------------------------------------------------------------
# Convenience optimizer over torch tensors
# --------------------------------------------------------------------------
class OKLS:
    """Online KL Shampoo over a list of matrix parameters (2-D (m, n) or 3-D
    (N, m, n); each parameter is one group of the C ABI).  Mirrors the README's
    optimizer interface: OKLS(params, lr, beta1, beta2, eps, weight_decay),
    .step(), .zero_grad(), .state_dict().  Gradients are read from p.grad
    (fp32, bf16 or fp16, as grad_dtype declares; checked against the
    parameter's shape and device) unless `grads` is passed to step().

    chunk_matrices = 0 runs every matrix in one chunk (the largest launches);
    with workspace_limit (bytes) set and chunk_matrices = 0, the largest
    chunk whose workspace fits the limit is chosen."""

    def __init__(self, params, lr=None, beta1=None, beta2=None, eps=None, weight_decay=None,
                 mode="okls", precision="fp16", grad_dtype=None, chunk_matrices=0, workspace_limit=None,
                 psi_seed=0, **cfg_overrides):
        import torch
        self.torch = torch
        self.params = list(params)
        if not self.params:
            raise ValueError("no parameters")
        hyper = HYPER_DEFAULTS["soap" if mode == "soap" else "okls"]
        lr = hyper["lr"] if lr is None else lr
        beta1 = hyper["beta1"] if beta1 is None else beta1
        beta2 = hyper["beta2"] if beta2 is None else beta2
        eps = hyper["eps"] if eps is None else eps
        weight_decay = hyper["weight_decay"] if weight_decay is None else weight_decay
        self.lr = float(lr)
        self.mode = mode
        if mode == "muon":
            cfg_overrides = {**MUON_DEFAULTS, **cfg_overrides}
        self.cfg = precision_config(precision, mode=MODE[mode], beta1=beta1, beta2=beta2, eps=eps,
                                    weight_decay=weight_decay, lr_peak=float(lr), chunk_matrices=chunk_matrices,
                                    **cfg_overrides)
        dev = self.params[0].device
        self.groups, self.state = [], []
        for p in self.params:
            if p.dtype != torch.float32 or not p.is_contiguous():
                raise ValueError("parameters must be contiguous fp32 tensors")
            shp = tuple(p.shape) if p.dim() == 3 else (1,) + tuple(p.shape)
            if len(shp) != 3:
                raise ValueError("parameters must be 2-D or 3-D")
            b, m, n = shp
            gdt = {torch.float32: OKLS_F32, torch.bfloat16: OKLS_BF16,
                   torch.float16: OKLS_F16}.get(grad_dtype or torch.float32)
            if gdt is None:
                raise ValueError("grad_dtype must be float32, bfloat16 or float16")
            self.groups.append((b, m, n, gdt))
            if mode == "muon":     # no factors or roots
                self.state.append(dict(M=torch.zeros(b, m, n, device=dev)))
            elif mode == "nystrom":   # low-rank factors U (d x r') and Lambda (r') per side
                r = self.cfg.nys_rank
                ka, kb = min(r + self.cfg.nys_oversample, m), min(r + self.cfg.nys_oversample, n)
                ra, rb = min(r, ka), min(r, kb)
                self.state.append(dict(M=torch.zeros(b, m, n, device=dev), Sa=torch.empty(b, ra, device=dev),
                                       Sb=torch.empty(b, rb, device=dev), Pa=torch.empty(b, m, ra, device=dev),
                                       Pb=torch.empty(b, n, rb, device=dev),
                                       PsiA=torch.zeros(b, m, ka, device=dev), PsiB=torch.zeros(b, n, kb, device=dev)))
            elif mode == "soap":   # factors, bases and both moments
                self.state.append(dict(M=torch.zeros(b, m, n, device=dev), V=torch.zeros(b, m, n, device=dev),
                                       Sa=torch.empty(b, m, m, device=dev), Sb=torch.empty(b, n, n, device=dev),
                                       Pa=torch.empty(b, m, m, device=dev), Pb=torch.empty(b, n, n, device=dev)))
            else:
                self.state.append(dict(M=torch.zeros(b, m, n, device=dev), Sa=torch.empty(b, m, m, device=dev),
                                       Sb=torch.empty(b, n, n, device=dev), Pa=torch.empty(b, m, m, device=dev),
                                       Pb=torch.empty(b, n, n, device=dev)))
        ws_bytes = workspace_size(self.cfg, self.groups)
        if ws_bytes == 0:
            raise OKLSError("okls_workspace_size", -1)
        if workspace_limit is not None and chunk_matrices == 0 and ws_bytes > workspace_limit:
            self.cfg.chunk_matrices, ws_bytes = fit_chunk(self.cfg, self.groups, int(workspace_limit))
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        self.handle = init(self.cfg, self.groups, self.workspace, self.stream)
        self.t = 0
        self.psi_seed = int(psi_seed)
        self._psi_gen = None
        init_state(self.handle, self._tensors(grads=None), self.stream)

    _GRAD_DTYPES = {OKLS_F32: "float32", OKLS_BF16: "bfloat16", OKLS_F16: "float16"}

    def _check_grad(self, i, g):
        """The library reads G as the dtype and shape declared at init: a
        mismatch would misread it or read past its end, so it is refused here."""
        b, m, n, gdt = self.groups[i]
        p = self.params[i]
        if g is None:
            raise ValueError(f"parameter {i} has no gradient")
        if g.dtype != getattr(self.torch, self._GRAD_DTYPES[gdt]):
            raise ValueError(f"gradient {i} is {g.dtype}, the optimizer was built for {self._GRAD_DTYPES[gdt]}")
        if tuple(g.shape) != tuple(p.shape):
            raise ValueError(f"gradient {i} has shape {tuple(g.shape)}, parameter {tuple(p.shape)}")
        if g.device != p.device:
            raise ValueError(f"gradient {i} is on {g.device}, parameter on {p.device}")

    def _tensors(self, grads, check=False):
        if grads is not None and len(grads) != len(self.params):
            raise ValueError(f"{len(grads)} gradients for {len(self.params)} parameters")
        per = []
        for i, p in enumerate(self.params):
            g = grads[i] if grads is not None else p.grad
            if check:
                self._check_grad(i, g)
            d = dict(self.state[i])
            d["W"] = p
            d["G"] = g.contiguous() if g is not None else None
            per.append(d)
        self._keep = per
        return tensors_array(per)

    def _draw_sketches(self, t):
        """Nystrom mode: the Gaussian matrices of a refresh step (t = 1, 1 + T, ...)
        are the method's random numbers, drawn here and passed to the library."""
        if self.mode != "nystrom" or (t - 1) % max(self.cfg.root_period, 1) != 0:
            return
        if self._psi_gen is None:
            self._psi_gen = self.torch.Generator(device=self.params[0].device).manual_seed(self.psi_seed)
        for s in self.state:
            for k in ("PsiA", "PsiB"):
                s[k].normal_(generator=self._psi_gen)

    def step(self, grads=None, lr=None):
        lr = self.lr if lr is None else float(lr)
        self.stream = self.torch.cuda.current_stream(self.params[0].device).cuda_stream
        self._draw_sketches(self.t + 1)
        tensors = self._tensors(grads, check=True)
        # the counter and the learning rate change only once the library has
        # accepted the step
        step(self.handle, tensors, self.t + 1, lr, self.stream)
        self.t += 1
        self.lr = lr

    def zero_grad(self):
        for p in self.params:
            p.grad = None

    def check_finite(self) -> bool:
        # G is not read by the scan; W stands in for its pointer
        return check_finite(self.handle, self._tensors(grads=list(self.params)), self.stream)

    def ns_residuals(self):
        """The Newton-Schulz residual of each root of the last step that
        recomputed them, per parameter: a list over the parameters of lists
        over the batch of [[a chain 0, a chain 1], [b chain 0, b chain 1]]."""
        flat = ns_residuals(self.handle, sum(g[0] for g in self.groups), self.stream)
        out, k = [], 0
        for (b, _, _, _) in self.groups:
            out.append(flat[k:k + b])
            k += b
        return out

    def state_dict(self):
        return {"t": self.t, "lr": self.lr, "lr_peak": self.cfg.lr_peak,
                "state": [{k: v.clone() for k, v in s.items()} for s in self.state]}

    def load_state_dict(self, sd):
        # lr_peak is part of the handle's configuration (the AdamC correction)
        if abs(float(sd["lr_peak"]) - float(self.cfg.lr_peak)) > 1e-6 * abs(float(self.cfg.lr_peak)):
            raise ValueError(f"state was saved with lr_peak {sd['lr_peak']}, this optimizer has {self.cfg.lr_peak}")
        # every tensor is checked before anything is copied, so a mismatched
        # checkpoint leaves this optimizer untouched
        if len(sd["state"]) != len(self.state):
            raise ValueError(f"state holds {len(sd['state'])} parameters, this optimizer has {len(self.state)}")
        for i, (dst, src) in enumerate(zip(self.state, sd["state"])):
            if set(src) != set(dst):
                raise ValueError(f"parameter {i}: state keys {sorted(src)}, expected {sorted(dst)}")
            for k, v in src.items():
                if tuple(v.shape) != tuple(dst[k].shape) or v.dtype != dst[k].dtype:
                    raise ValueError(f"parameter {i} {k}: {tuple(v.shape)} {v.dtype}, "
                                     f"expected {tuple(dst[k].shape)} {dst[k].dtype}")
        self.t = int(sd["t"])
        self.lr = float(sd["lr"])
        for dst, src in zip(self.state, sd["state"]):
            for k, v in src.items():
                dst[k].copy_(v)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.okls_destroy(h)
            self.handle = None
