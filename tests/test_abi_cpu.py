"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/rk.h, the ctypes layouts match the C structs, and every
host-side validation path returns its status before any HIP call."""

import ctypes as C
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from masked_attention_amd import _rk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rk.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_rk.LIB_PATH):
        pytest.skip("librk.so not built")
    return _rk.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(rk_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_operations():
    names = _declared_functions()
    for n in ("rk_mask_plan", "rk_time_rope", "rk_masked_attn_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    declared = {f[0] for f in _rk.FUNCTIONS}
    assert declared == set(names)
    # and the dynamic symbol table has them as C (unmangled) symbols
    out = subprocess.run(["nm", "-D", "--defined-only", _rk.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_abi_version_and_status_strings(lib):
    assert lib.rk_abi_version() == _rk.RK_ABI_VERSION
    for s in range(7):
        assert len(lib.rk_status_string(s)) > 0


def test_ctypes_layouts_match_c_structs():
    fields = {name: [f[0] for f in cls._fields_] for name, cls in _rk.STRUCTS.items()}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void){']
    for name, fl in fields.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for f in fl:
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    for name, cls in _rk.STRUCTS.items():
        assert int(got[name]) == C.sizeof(cls), name
        for f in fields[name]:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, f"{name}.{f}"


def _batch(offs, T=None):
    offs = np.asarray(offs, np.int32)
    b = _rk.sized(_rk.rk_batch, num_requests=len(offs) - 1,
                  total_tokens=int(offs[-1]) if T is None else T,
                  req_offsets_host=offs.ctypes.data, req_offsets_dev=0x1000,
                  seg_kind_dev=0x2000, timestamps_dev=0x3000, anchors_dev=0x4000)
    return b, offs


def test_workspace_size_validation(lib):
    n = C.c_size_t()
    b, keep = _batch([0, 10, 10, 300])
    assert lib.rk_plan_workspace_size(C.byref(b), 4, C.byref(n)) == _rk.RK_OK
    assert n.value > 0 and n.value % 256 == 0
    small = n.value
    b2, keep2 = _batch([0, 20000, 40000])
    assert lib.rk_plan_workspace_size(C.byref(b2), 4, C.byref(n)) == _rk.RK_OK
    assert n.value > small
    # 2 requests x 157 q-tiles x 313 k-tiles: class + count + csr + cls >= 10 bytes per tile
    assert n.value >= 2 * 157 * 313 * 10
    bad = [
        ([1, 10], None),          # offsets must start at 0
        ([0, 10, 5], None),       # decreasing
        ([0, 10, 20], 19),        # last offset != total_tokens
    ]
    for offs, T in bad:
        bb, k = _batch(offs, T)
        assert lib.rk_plan_workspace_size(C.byref(bb), 4, C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_plan_workspace_size(C.byref(b), 0, C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_plan_workspace_size(None, 1, C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    b3, k3 = _batch([0, 10])
    b3.struct_size = 8
    assert lib.rk_plan_workspace_size(C.byref(b3), 1, C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    b4, k4 = _batch([0, 10])
    b4.seg_kind_dev = None
    assert lib.rk_plan_workspace_size(C.byref(b4), 1, C.byref(n)) == _rk.RK_ERR_INVALID_ARG


def test_mask_plan_host_errors(lib):
    b, keep = _batch([0, 100, 300])
    n = C.c_size_t()
    assert lib.rk_plan_workspace_size(C.byref(b), 2, C.byref(n)) == _rk.RK_OK
    h = C.c_void_p()
    m = _rk.sized(_rk.rk_mask_params, delay=3600, window=0)
    # too small (pointer is never dereferenced: the size check comes first)
    assert lib.rk_mask_plan(C.byref(b), C.byref(m), 2, C.c_void_p(1 << 20), n.value - 256,
                            C.byref(h), None) == _rk.RK_ERR_WORKSPACE_TOO_SMALL
    assert h.value is None
    # misaligned / NULL workspace
    assert lib.rk_mask_plan(C.byref(b), C.byref(m), 2, C.c_void_p((1 << 20) + 8), n.value,
                            C.byref(h), None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_mask_plan(C.byref(b), C.byref(m), 2, None, n.value, C.byref(h),
                            None) == _rk.RK_ERR_INVALID_ARG
    for bad in (dict(delay=-1), dict(window=-3), dict(flags=8), dict(global_tail=-1),
                dict(flags=_rk.RK_QUERY_CANDIDATES_ONLY | 8),
                dict(flags=_rk.RK_QUERY_CANDIDATES_ONLY | _rk.RK_PLAN_BACKWARD)):
        mb = _rk.sized(_rk.rk_mask_params, **bad)
        assert lib.rk_mask_plan(C.byref(b), C.byref(mb), 2, C.c_void_p(1 << 20), n.value,
                                C.byref(h), None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_mask_plan(C.byref(b), None, 2, C.c_void_p(1 << 20), n.value, C.byref(h),
                            None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_mask_plan(C.byref(b), C.byref(m), 2, C.c_void_p(1 << 20), n.value, None,
                            None) == _rk.RK_ERR_INVALID_ARG


def test_time_rope_host_errors(lib):
    b, keep = _batch([0, 100])
    rp = _rk.sized(_rk.rk_rope_params, phi_min=1e-4, dt_max=31536000.0, base=6e5)
    args = lambda **kw: dict(dict(b=C.byref(b), r=C.byref(rp), x=C.c_void_p(1 << 20),
                                  y=C.c_void_p(1 << 21), dt=_rk.RK_BF16, H=2, d=64,
                                  ist=128, ish=64, ost=128, osh=64), **kw)

    def call(a):
        return lib.rk_time_rope(a["b"], a["r"], a["x"], a["y"], a["dt"], a["H"], a["d"], a["ist"],
                                a["ish"], a["ost"], a["osh"], None)

    assert call(args(d=63)) == _rk.RK_ERR_UNSUPPORTED
    assert call(args(d=256)) == _rk.RK_ERR_UNSUPPORTED
    assert call(args(H=0)) == _rk.RK_ERR_INVALID_ARG
    assert call(args(dt=7)) == _rk.RK_ERR_INVALID_ARG
    assert call(args(x=None)) == _rk.RK_ERR_INVALID_ARG
    assert call(args(ist=-1)) == _rk.RK_ERR_INVALID_ARG
    assert call(args(y=C.c_void_p(1 << 20), ost=256)) == _rk.RK_ERR_INVALID_ARG  # in place, strides differ
    for bad in (dict(phi_min=0.0), dict(dt_max=-1.0), dict(base=float("nan")), dict(kinds=16)):
        rb = _rk.sized(_rk.rk_rope_params, **dict(dict(phi_min=1e-4, dt_max=1.0, base=2.0), **bad))
        assert call(args(r=C.byref(rb))) == _rk.RK_ERR_INVALID_ARG


def test_attention_host_errors_without_plan(lib):
    a = _rk.sized(_rk.rk_attn_args, dtype=_rk.RK_BF16, num_heads=1, d_head=64)
    assert lib.rk_masked_attn_fwd(None, C.byref(a), None) == _rk.RK_ERR_INVALID_ARG
    n = C.c_size_t()
    assert lib.rk_attn_workspace_size(None, C.byref(a), C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    t = _rk.sized(_rk.rk_plan_totals)
    assert lib.rk_plan_stats(None, C.byref(t), None) == _rk.RK_ERR_INVALID_ARG
    info = _rk.sized(_rk.rk_plan_info)
    assert lib.rk_plan_get_info(None, C.byref(info)) == _rk.RK_ERR_INVALID_ARG
    lib.rk_plan_destroy(None)  # no-op
    ab = _rk.sized(_rk.rk_attn_bwd_args, dtype=_rk.RK_BF16, num_heads=1, d_head=64)
    assert lib.rk_masked_attn_bwd(None, C.byref(ab), None) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_attn_bwd_workspace_size(None, C.byref(ab), C.byref(n)) == _rk.RK_ERR_INVALID_ARG
    assert lib.rk_masked_attn_bwd(None, None, None) == _rk.RK_ERR_INVALID_ARG
