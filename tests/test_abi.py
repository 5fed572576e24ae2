"""The C-ABI library loads, exports every symbol include/okls.h declares,
and validates its arguments on the host (no GPU needed: every call here
returns before touching the device)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from kronecker_factored_second_amd import okls
from oracle import okls_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(okls.LIB_PATH):
        pytest.skip("libokls.so not built")
    return okls.load()


def test_exports_every_declared_symbol():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "okls.h")).read()
    declared = set(re.findall(r"\b(okls_[a-z_]+)\s*\(", header))
    assert declared == set(okls.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_binding_struct_layouts_match_header(tmp_path):
    """sizeof and field offsets of the ABI structs, from the C compiler on
    include/okls.h, equal the ctypes mirrors of the binding."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"okls_config": okls.Config, "okls_group_desc": okls.GroupDesc,
               "okls_group_tensors": okls.GroupTensors, "okls_profile_stats": okls.ProfileStats}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "okls.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


def test_default_config_matches_pages():
    _lib()
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "okls_defaults.json")))
    c = okls.default_config()
    assert c.ns_steps == g["ns_steps"]
    for k in ("beta1", "beta2", "eps", "weight_decay"):
        assert getattr(c, k) == pytest.approx(g[k], rel=1e-6)
    assert c.lr_peak == pytest.approx(g["lr"], rel=1e-6)


def test_ns_coefficients_match_oracle():
    _lib()
    for floor, steps in [(1e-3, 10), (0.05, 6), (1e-4, 16)]:
        c = okls.default_config(ns_floor=floor, ns_steps=steps)
        a, b = okls.ns_coefficients(c)
        ref, _ = O.ns_coefficients(float(np.float32(floor)), steps)
        np.testing.assert_allclose(a, [x for x, _ in ref], rtol=1e-12)
        np.testing.assert_allclose(b, [y for _, y in ref], rtol=1e-12)


def test_workspace_size_validation():
    _lib()
    c = okls.default_config()
    assert okls.workspace_size(c, [(1, 128, 256, 0)]) > 0
    assert okls.workspace_size(c, [(0, 128, 256, 0)]) == 0        # empty batch
    assert okls.workspace_size(c, [(1, 0, 256, 0)]) == 0
    assert okls.workspace_size(c, [(1, 40000, 8, 0)]) == 0        # beyond the maximum side
    assert okls.workspace_size(c, [(1, 8, 8, 7)]) == 0            # bad dtype
    for gdt in (okls.OKLS_F32, okls.OKLS_BF16, okls.OKLS_F16):    # fp32, bf16, fp16 gradients
        assert okls.workspace_size(c, [(1, 128, 256, gdt)]) > 0
    assert okls.workspace_size(c, [(1, 8, 8, 0)] * 17) == 0       # too many groups
    for k in ("eps_convex", "decay_after", "shape_scale", "ns_classical"):   # the reading switches are 0 or 1
        assert okls.workspace_size(okls.default_config(**{k: 2}), [(1, 8, 8, 0)]) == 0
        assert okls.workspace_size(okls.default_config(**{k: 1}), [(1, 8, 8, 0)]) > 0
    d = okls.default_config()
    assert (d.eps_convex, d.decay_after, d.shape_scale, d.ns_classical) == (0, 0, 1, 0)
    a, b = okls.ns_coefficients(okls.default_config(ns_classical=1, ns_steps=12))
    assert a == [1.5] * 12 and b == [-0.5] * 12
    bad = okls.default_config(ns_steps=1)
    assert okls.workspace_size(bad, [(1, 8, 8, 0)]) == 0
    one = okls.workspace_size(c, [(1, 1024, 1024, 1)])
    four = okls.workspace_size(c, [(4, 1024, 1024, 1)])
    chunked = okls.workspace_size(okls.default_config(chunk_matrices=1), [(4, 1024, 1024, 1)])
    assert four > 3 * (one // 2) and chunked < four
    split = okls.workspace_size(okls.precision_config("fp32"), [(1, 1024, 1024, 1)])
    assert split > one


def test_host_side_errors_before_any_launch():
    lib = _lib()
    c = okls.default_config()
    groups = (okls.GroupDesc * 1)(okls.GroupDesc(1, 64, 64, 0))
    h = ctypes.c_void_p()
    assert lib.okls_init(ctypes.byref(h), ctypes.byref(c), 1, groups, None, 1 << 30, None) == -4
    assert lib.okls_init(ctypes.byref(h), ctypes.byref(c), 1, groups, ctypes.c_void_p(4096 + 8), 1 << 30, None) == -4
    assert lib.okls_init(ctypes.byref(h), ctypes.byref(c), 1, groups, ctypes.c_void_p(4096), 16, None) == -4
    assert lib.okls_init(ctypes.byref(h), None, 1, groups, ctypes.c_void_p(4096), 1 << 30, None) == -1
    assert lib.okls_init(None, ctypes.byref(c), 1, groups, ctypes.c_void_p(4096), 1 << 30, None) == -1
    assert lib.okls_step(None, None, 1, ctypes.c_float(0.1), None) == -1
    assert lib.okls_init_state(None, None, None) == -1
    assert lib.okls_destroy(None) == -1
    assert okls.status_string(-4).startswith("workspace")
    assert okls.status_string(0) == "ok"


def test_fault_injection_hook(monkeypatch):
    """OKLS_FAULT=<call> makes that call fail with OKLS_ERR_HIP after its
    argument checks, so the binding's error path runs without a GPU."""
    lib = _lib()
    monkeypatch.setenv("OKLS_FAULT", "okls_init")
    c = okls.default_config()
    groups = (okls.GroupDesc * 1)(okls.GroupDesc(1, 64, 64, 0))
    h = ctypes.c_void_p()
    assert lib.okls_init(ctypes.byref(h), ctypes.byref(c), 1, groups, ctypes.c_void_p(4096), 1 << 40, None) == -5
    assert h.value is None


def test_binding_raises_without_library(tmp_path):
    saved = okls._lib
    okls._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            okls.load(str(tmp_path / "nope.so"))
    finally:
        okls._lib = saved


def test_muon_plans_validate_on_the_host():
    """Muon mode (polar iteration of the momentum) plans and validates its
    descriptors for wide, tall, ragged and tiny shapes on both paths; the
    iteration needs at least two steps."""
    for prec in ("fp16", "fp32"):
        cfg = okls.precision_config(prec, mode=okls.MODE["muon"], **okls.MUON_DEFAULTS)
        for groups in ([(2, 96, 160, 0)], [(1, 200, 72, 0), (3, 33, 40, 1)], [(1, 1, 7, 0)],
                       [(4, 1024, 1024, 1), (2, 2816, 1024, 1), (1, 1024, 2816, 1)]):
            assert okls.workspace_size(cfg, groups) > 0, (prec, groups)
        cfg.ns_steps = 1
        assert okls.workspace_size(cfg, [(1, 64, 80, 0)]) == 0
