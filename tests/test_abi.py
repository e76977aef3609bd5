"""The C ABI loads, exports every declared symbol, and rejects bad arguments on the
host before any device work (CPU only: no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

import varlen_causal_attention_amd as vlca
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "varlen_causal_attn.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s+(varlen_causal_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(vlca.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = vlca.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", vlca.library_path()], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = set(ln.split()[-1] for ln in nm.stdout.splitlines() if ln.strip())
        for name in declared_functions():
            assert name in exported, name


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void) {{ return varlen_causal_attn_tile_rows() == 64 ? 0 : 1; }}\n'
    res = subprocess.run(["gcc", "-std=c11", "-fsyntax-only", "-x", "c", "-"], input=src, capture_output=True,
                         text=True)
    assert res.returncode == 0, res.stderr


def test_constants_and_strings():
    assert vlca.tile_rows() == 64
    assert vlca.strerror(0) == "success"
    for code in range(-15, 0):
        assert vlca.strerror(code) != "unknown error code"
    assert vlca.strerror(-99) == "unknown error code"


def test_worklist_capacity():
    assert vlca.worklist_capacity(60, 452) == 60 * 8
    assert vlca.worklist_capacity(0, 0) == 0
    assert vlca.worklist_capacity(1000, 4096) == 1000 * 64
    with pytest.raises(vlca.VlcaError) as e:
        vlca.worklist_capacity(-1, 10)
    assert e.value.code == -2
    with pytest.raises(vlca.VlcaError) as e:
        vlca.worklist_capacity(10, 262145)
    assert e.value.code == -6
    with pytest.raises(vlca.VlcaError) as e:
        vlca.worklist_capacity(600000, 262144)  # > 2^31 items
    assert e.value.code == -6


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _fwd(qkv=FAKE, cu=FAKE, U=4, ms=40, H=8, D=64, scale=0.125, out=FAKE * 2):
    return vlca.library().varlen_causal_attn_fwd(qkv, cu, U, ms, H, D, ctypes.c_float(scale), out, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(U=-1), -2),
    (dict(ms=-5), -2),
    (dict(D=128), -3),
    (dict(D=32), -3),
    (dict(H=0), -4),
    (dict(H=70000), -4),
    (dict(scale=float("nan")), -5),
    (dict(scale=float("inf")), -5),
    (dict(scale=0.0), -5),
    (dict(scale=-0.125), -5),
    (dict(ms=262145), -6),
    (dict(qkv=None), -1),
    (dict(cu=None), -1),
    (dict(out=None), -1),
    (dict(out=FAKE), -8),
])
def test_fwd_rejects_bad_arguments_before_device_work(kwargs, code):
    assert _fwd(**kwargs) == code


def test_fwd_zero_users_or_zero_length_is_a_noop():
    # No device is touched: these return before any HIP call.
    assert _fwd(qkv=None, cu=None, out=None, U=0) == 0
    assert _fwd(ms=0) == 0


def test_build_worklist_and_fwd_worklist_validation():
    lib = vlca.library()
    assert lib.varlen_causal_attn_build_worklist(FAKE, 4, 40, None, 5000, FAKE, None) == -1
    assert lib.varlen_causal_attn_build_worklist(FAKE, 4, 40, FAKE, 5000, None, None) == -1
    assert lib.varlen_causal_attn_build_worklist(None, 4, 40, FAKE, 5000, FAKE, None) == -1
    assert lib.varlen_causal_attn_build_worklist(FAKE, 4, 40, FAKE, 3, FAKE, None) == -7
    assert lib.varlen_causal_attn_build_worklist(FAKE, -4, 40, FAKE, 9999, FAKE, None) == -2
    f = lib.varlen_causal_attn_fwd_worklist
    c = ctypes.c_float(0.125)
    assert f(FAKE, FAKE, 4, 40, 8, 64, c, None, 5000, FAKE, FAKE * 2, None) == -1
    assert f(FAKE, FAKE, 4, 40, 8, 64, c, FAKE, 5000, None, FAKE * 2, None) == -1
    assert f(FAKE, FAKE, 4, 40, 8, 64, c, FAKE, 3, FAKE, FAKE * 2, None) == -7
    assert f(FAKE, FAKE, 4, 40, 8, 96, c, FAKE, 5000, FAKE, FAKE * 2, None) == -3
    assert f(None, None, 0, 40, 8, 64, c, None, 0, None, None, None) == 0


def test_single_kernel_query_validation():
    # Size checks run before any HIP call.
    f = vlca.library().varlen_causal_attn_single_kernel
    flag = ctypes.c_int(7)
    assert f(-1, 40, 8, ctypes.byref(flag)) == -2
    assert f(4, 262145, 8, ctypes.byref(flag)) == -6
    assert f(4, 40, 0, ctypes.byref(flag)) == -4
    assert f(4, 40, 8, None) == -1
    assert flag.value == 7


def _tramp_args(qkv=FAKE, cu=FAKE, U=4, ms=40, H=8, D=64, scale=0.125, out=FAKE * 2):
    return (0 if qkv is None else qkv, 0 if cu is None else cu, U, ms, H, D, scale, 0 if out is None else out, 0)


def test_call_module_is_built_and_bound():
    assert vlca.call_module() is not None, "the CPython call module was not built"


@pytest.mark.parametrize("kwargs", [
    dict(U=-1), dict(D=128), dict(H=0), dict(scale=float("nan")), dict(scale=0.0), dict(ms=262145),
    dict(qkv=None), dict(out=None), dict(out=FAKE), dict(U=0, qkv=None, cu=None, out=None), dict(ms=0),
])
def test_call_module_passes_arguments_like_ctypes(kwargs):
    # Both routes reach the same validation (no device work): equal return codes.
    m = vlca.call_module()
    a = _tramp_args(**kwargs)
    assert m.fwd(*a) == _fwd(**kwargs)
    w = a[:7] + (FAKE, 5000, FAKE) + a[7:]  # items, capacity, count before out, stream
    ref = vlca.library().varlen_causal_attn_fwd_worklist(*w[:6], ctypes.c_float(w[6]), *w[7:])
    assert m.fwd_worklist(*w) == ref


def test_call_module_rejects_bad_python_arguments():
    m = vlca.call_module()
    with pytest.raises(TypeError):
        m.fwd(*_tramp_args()[:8])
    with pytest.raises(TypeError):
        m.fwd(*_tramp_args(U="4"))
    with pytest.raises(OverflowError):
        m.fwd(*_tramp_args(U=2**40))
    with pytest.raises(TypeError):
        m.fwd_worklist(*_tramp_args())
