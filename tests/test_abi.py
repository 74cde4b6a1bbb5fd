"""The C-ABI library: it builds for gfx950, loads, exports every function
include/specverify.h declares, and rejects bad arguments on the host before
any GPU work (no compute call is made here)."""

import ctypes
import os
import re
import subprocess

import pytest

from rejection_sampling_verifier_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from rejection_sampling_verifier_amd import build
        build.build(verbose=False)
    return binding.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", src)))


def test_header_declares_the_interface():
    names = declared_functions()
    assert "spec_verify" in names and "spec_verify_probe" in names and "spec_smc_step" in names
    assert "spec_hispec_verify" in names and "spec_greedy_verify" in names
    assert set(names) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_holds_gfx950_code():
    out = subprocess.run(["strings", binding.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "gfx950" in out


def test_abi_version_and_messages(lib):
    assert lib.spec_verify_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert len(lib.spec_verify_strerror(code)) > 3


def _call(lib, B=2, K=3, V=100, dtype=0, T=1.0, top_p=1.0, tP=None, dP=None, tdata=0x1000, ddata=0x2000,
          tokens=0x3000, out=0x4000, outn=0x5000, dtype_d=None, stride=(0, 0)):
    t = binding.SvLogits(tdata, dtype, B, K + 1 if tP is None else tP, V, (K + 1) * V + stride[0], V + stride[1])
    d = binding.SvLogits(ddata, dtype if dtype_d is None else dtype_d, B, K if dP is None else dP, V, K * V, V)
    return lib.spec_verify(ctypes.byref(t), ctypes.byref(d), ctypes.c_void_p(tokens), ctypes.c_void_p(None),
                           ctypes.c_float(T), ctypes.c_float(top_p), ctypes.c_uint64(0), ctypes.c_void_p(out),
                           ctypes.c_void_p(outn), ctypes.c_void_p(None))


@pytest.mark.parametrize("kw,code", [
    (dict(tdata=0), -1), (dict(tokens=0), -1), (dict(out=0), -1),
    (dict(dtype=7), -3), (dict(dtype_d=1), -3),
    (dict(K=0), -2), (dict(K=17), -2), (dict(B=0), -2), (dict(V=0), -2), (dict(dP=2), -2), (dict(tP=3), -2),
    (dict(T=0.0), -1), (dict(T=-1.0), -1), (dict(T=float("nan")), -1), (dict(T=float("inf")), -1),
    (dict(T=1e-45), -1),
    (dict(top_p=0.0), -1), (dict(top_p=1.5), -1), (dict(top_p=float("nan")), -1),
    (dict(tdata=0x1002), -6), (dict(dtype=1, dtype_d=1, tdata=0x1001), -6), (dict(tokens=0x3002), -6),
    (dict(stride=(-2 * 400, 0)), -1),
    (dict(V=(1 << 21) + 1), -2), (dict(V=(1 << 24) + 1), -2),
])
def test_host_validation(lib, kw, code):
    assert _call(lib, **kw) == code


def _smc(lib, N=4, K=2, V=64, T=1.0, ess=0.5, tdata=0x1000, ddata=0x2000, tokens=0x3000, lw=0x4000, bonus=0x5000,
         lwo=0x6000, anc=0x7000, e=0x8000, rs=0x9000, tP=None):
    t = binding.SvLogits(tdata, 0, N, K + 1 if tP is None else tP, V, (K + 1) * V, V)
    d = binding.SvLogits(ddata, 0, N, K, V, K * V, V)
    v = ctypes.c_void_p
    return lib.spec_smc_step(ctypes.byref(t), ctypes.byref(d), v(tokens), v(lw), ctypes.c_float(T),
                             ctypes.c_double(ess), ctypes.c_uint64(0), v(bonus), v(lwo), v(anc), v(e), v(rs), v(None))


@pytest.mark.parametrize("kw,code", [
    (dict(lw=0), -1), (dict(bonus=0), -1), (dict(lwo=0), -1), (dict(anc=0), -1), (dict(e=0), -1), (dict(rs=0), -1),
    (dict(tokens=0), -1), (dict(ess=float("nan")), -1), (dict(T=0.0), -1),
    (dict(lw=0x4004), -6), (dict(lwo=0x6004), -6), (dict(e=0x8004), -6), (dict(anc=0x7002), -6),
    (dict(K=0), -2), (dict(K=17), -2), (dict(N=0), -2), (dict(tP=2), -2), (dict(V=(1 << 21) + 1), -2),
])
def test_smc_host_validation(lib, kw, code):
    assert _smc(lib, **kw) == code


def _hispec(lib, B=3, K=2, V=64, fP=None, iP=None, T=1.0, fdata=0x1000, idata=0x2000, ddata=0x3000, tokens=0x4000,
            out=0x5000, outn=0x6000, outn1=0x7000, dtype_f=0):
    f = binding.SvLogits(fdata, dtype_f, B, K + 2 if fP is None else fP, V, (K + 2) * V, V)
    i = binding.SvLogits(idata, 0, B, K + 1 if iP is None else iP, V, (K + 1) * V, V)
    d = binding.SvLogits(ddata, 0, B, K, V, K * V, V)
    v = ctypes.c_void_p
    return lib.spec_hispec_verify(ctypes.byref(f), ctypes.byref(i), ctypes.byref(d), v(tokens), v(None),
                                  ctypes.c_float(T), ctypes.c_float(1.0), ctypes.c_uint64(0), v(out), v(outn),
                                  v(outn1), v(None))


@pytest.mark.parametrize("kw,code", [
    (dict(out=0), -1), (dict(outn=0), -1), (dict(tokens=0), -1), (dict(fdata=0), -1), (dict(T=0.0), -1),
    (dict(fP=3), -2), (dict(iP=2), -2), (dict(K=15 + 1), -2), (dict(dtype_f=1), -3), (dict(V=(1 << 21) + 1), -2),
    (dict(out=0x5002), -6), (dict(outn1=0x7002), -6),
])
def test_hispec_host_validation(lib, kw, code):
    assert _hispec(lib, **kw) == code


def _greedy(lib, B=3, K=2, V=64, k=5, tdata=0x1000, tokens=0x4000, out=0x5000, outn=0x6000, topk=0x7000, dtype=0):
    t = binding.SvLogits(tdata, dtype, B, K + 1, V, (K + 1) * V, V)
    v = ctypes.c_void_p
    return lib.spec_greedy_verify(ctypes.byref(t), v(tokens), v(None), ctypes.c_int32(k), v(out), v(outn), v(topk),
                                  v(None))


@pytest.mark.parametrize("kw,code", [
    (dict(out=0), -1), (dict(outn=0), -1), (dict(tokens=0), -1), (dict(tdata=0), -1), (dict(topk=0), -1),
    (dict(k=-1), -1), (dict(k=65), -1), (dict(K=0), -2), (dict(K=17), -2), (dict(dtype=5), -3),
    (dict(V=(1 << 24) + 1), -2),
    (dict(out=0x5002), -6), (dict(topk=0x7001), -6),
])
def test_greedy_host_validation(lib, kw, code):
    assert _greedy(lib, **kw) == code


def _produce(lib, B=3, P=4, K=2, V=64, tdata=0x1000, out=0x5000, osb=None, osp=None, tokens=0x6000, dtype=1):
    t = binding.SvLogits(tdata, dtype, B, P, V, P * V, V)
    v = ctypes.c_void_p
    return lib.spec_draft_produce(ctypes.byref(t), ctypes.c_int32(K), ctypes.c_uint64(1), v(out),
                                  ctypes.c_int64(K * V if osb is None else osb), ctypes.c_int64(V if osp is None else osp),
                                  v(tokens), v(None))


@pytest.mark.parametrize("kw,code", [
    (dict(out=0), -1), (dict(tokens=0), -1), (dict(tdata=0), -1), (dict(osb=-1), -1), (dict(osp=-5), -1),
    (dict(K=0), -2), (dict(K=5), -2), (dict(B=0), -2), (dict(V=0), -2), (dict(dtype=7), -3),
    (dict(out=0x5001), -6), (dict(tokens=0x6002), -6), (dict(tdata=0x1001), -6),
])
def test_produce_host_validation(lib, kw, code):
    assert _produce(lib, **kw) == code


def _noalloc(lib, B=2, K=3, V=100):
    t = binding.SvLogits(0x1000, 0, B, K + 1, V, (K + 1) * V, V)
    d = binding.SvLogits(0x2000, 0, B, K, V, K * V, V)
    v = ctypes.c_void_p
    return lib.spec_verify_noalloc(ctypes.byref(t), ctypes.byref(d), v(0x3000), v(None), ctypes.c_float(1.0),
                                   ctypes.c_float(1.0), ctypes.c_uint64(0), v(0x4000), v(0x5000), v(None))


def test_forced_launch_failure_returns_ehip(lib, monkeypatch):
    # SPECVERIFY_FAIL_LAUNCH makes every entry point fail as a failed kernel
    # launch does, before it touches the device: SV_EHIP, with the message
    monkeypatch.setenv("SPECVERIFY_FAIL_LAUNCH", "1")
    assert _call(lib) == -4
    assert b"SPECVERIFY_FAIL_LAUNCH" in lib.spec_verify_strerror(-4)
    assert _call(lib, dtype=1, top_p=0.9) == -4
    assert _smc(lib) == -4
    assert _hispec(lib) == -4
    assert _greedy(lib) == -4
    assert _produce(lib) == -4
    assert _noalloc(lib) == -4
    # host-checked argument errors still come first
    assert _call(lib, tdata=0) == -1
    monkeypatch.delenv("SPECVERIFY_FAIL_LAUNCH")
    assert _call(lib, tdata=0) == -1


def test_release_without_scratch_is_harmless(lib):
    # nothing allocated (no GPU call was made): releasing twice does nothing
    lib.spec_verify_release()
    lib.spec_verify_release()
    assert lib.spec_verify_abi_version() == 1
