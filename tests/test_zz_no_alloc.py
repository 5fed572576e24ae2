"""okls_init_static (the library's static device scratch as the workspace,
for callers that cannot allocate) against okls_init with a workspace: two
handles in a row on the same scratch, the second with smaller groups, each
stepped through the C ABI; states bit-identical to the workspace handle's,
and within the fp64 oracle's bounds like any step."""
import ctypes

import numpy as np
import pytest

from kronecker_factored_second_amd import okls
from oracle import okls_oracle as O

pytestmark = pytest.mark.gpu


def _state(groups, seed):
    import torch
    rng = np.random.default_rng(seed)
    out = []
    for (b, m, n, _) in groups:
        out.append(dict(W=torch.tensor(0.01 * rng.standard_normal((b, m, n)), dtype=torch.float32, device="cuda:0"),
                        M=torch.zeros(b, m, n, device="cuda:0"), Sa=torch.empty(b, m, m, device="cuda:0"),
                        Sb=torch.empty(b, n, n, device="cuda:0"), Pa=torch.empty(b, m, m, device="cuda:0"),
                        Pb=torch.empty(b, n, n, device="cuda:0")))
    return out


def _run(groups, static, steps, seed):
    import torch
    cfg = okls.precision_config("fp16")
    stream = torch.cuda.current_stream().cuda_stream
    st = _state(groups, seed)
    ws = None
    if static:
        h = okls.init_static(cfg, groups, stream)
    else:
        ws = torch.empty(okls.workspace_size(cfg, groups), dtype=torch.uint8, device="cuda:0")
        h = okls.init(cfg, groups, ws, stream)
    grads = []
    for t in range(1, steps + 1):
        gs = [torch.tensor((0.02 * np.random.default_rng([seed, t, gi]).standard_normal((b, m, n))).astype(np.float32),
                           device="cuda:0") for gi, (b, m, n, _) in enumerate(groups)]
        grads.append(gs)
        for d, g in zip(st, gs):
            d["G"] = g
        if t == 1:
            okls.init_state(h, okls.tensors_array(st), stream)
        okls.step(h, okls.tensors_array(st), t, cfg.lr_peak, stream)
    torch.cuda.synchronize()
    okls.destroy(h)
    return [{k: v.cpu().numpy().copy() for k, v in d.items() if k != "G"} for d in st], grads


def test_static_scratch_matches_workspace_two_calls_in_a_row():
    pytest.importorskip("torch")
    for groups, seed in (([(2, 96, 160, 0), (1, 200, 72, 0)], 3), ([(1, 40, 33, 0)], 4)):
        a, _ = _run(groups, True, 3, seed)
        b, _ = _run(groups, False, 3, seed)
        for da, db in zip(a, b):
            for k in da:
                assert np.array_equal(da[k], db[k]), (groups, k)
        for d in a:
            assert all(np.isfinite(v).all() for v in d.values())


def test_static_scratch_refuses_groups_beyond_its_size():
    import torch
    cfg = okls.precision_config("fp16")
    groups = [(1, 4096, 4096, 0)]
    assert okls.workspace_size(cfg, groups) > okls.STATIC_SCRATCH_BYTES
    h = ctypes.c_void_p()
    st = okls.load().okls_init_static(ctypes.byref(h), ctypes.byref(cfg), 1, okls._groups_array(groups),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -4 and not h.value
