"""Host-side checks of liborbit.so that need no GPU: exports, the fp64
Lloyd-Max fitter against the oracle's independent fitter, and argument
validation (which runs before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import rotation_bit_ptq_amd as rbp
    return rbp


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "orbit.h")).read()
    declared = set(re.findall(r"\b(orbit_[a-z0-9_]+)\s*\(", header))
    assert len(declared) >= 9
    lib = ctypes.CDLL(_lib().LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 6, 8])
def test_fitter_agrees_with_oracle(bits):
    # two different solvers (Newton on thresholds here, fixed-point + MINPACK
    # in the oracle) must land on the unique Lloyd-Max fixed point
    cb = _lib().Codebook(3072, bits)
    ref = oracle.lloyd_max_gaussian(2 ** bits)
    np.testing.assert_allclose(cb.centroids_f64, ref["centroids"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(cb.thresholds_f64, ref["thresholds"], rtol=0, atol=1e-11)
    assert abs(cb.mse - ref["distortion"]) < 1e-12
    # float32 tables are the nearest floats of the fp64 values
    np.testing.assert_array_equal(cb.centroids, ref["centroids"].astype(np.float32))
    np.testing.assert_array_equal(cb.thresholds, ref["thresholds"].astype(np.float32))
    assert cb.thresholds[2 ** (bits - 1) - 1] == 0.0


@pytest.mark.parametrize("d", [3, 4, 16, 64, 3072, 12288])
@pytest.mark.parametrize("bits", [1, 2, 4, 6, 8])
def test_sphere_fitter_agrees_with_oracle(d, bits):
    # the library evaluates the incomplete beta with its own continued
    # fraction and solves by Newton; the oracle calls scipy's betaincc and
    # MINPACK: both must land on the unique (f_d is log-concave for d >= 3)
    # fixed point.  Evaluated with 40-digit functions (mpmath), both fits
    # leave a residual of ~4e-12 (the tails are good to ~3e-15 relative), and
    # the fixed point's condition number grows like L^2 for L levels (its
    # slowest Lloyd modes), so the two solutions may differ by ~1e-12 L^2;
    # the float32 tables the kernels read may differ by one ulp at most.
    L = 2 ** bits
    cb = _lib().Codebook(d, bits, marginal="sphere")
    ref = oracle.lloyd_max_sphere(L, d)
    np.testing.assert_allclose(cb.centroids_f64, ref["centroids"], rtol=0, atol=1e-12 * L * L)
    np.testing.assert_allclose(cb.thresholds_f64, ref["thresholds"], rtol=0, atol=1e-12 * L * L)
    assert abs(cb.mse - ref["distortion"]) < 1e-11
    for got, want in ((cb.centroids, ref["centroids"]), (cb.thresholds, ref["thresholds"])):
        ulps = np.abs(got.view(np.int32).astype(np.int64)
                      - want.astype(np.float32).view(np.int32).astype(np.int64))
        assert ulps.max() <= 1
    assert cb.thresholds[2 ** (bits - 1) - 1] == 0.0
    assert cb.marginal == "sphere" and cb.d == d


def test_sphere_fit_errors():
    cb = _lib()._Codebook()
    assert _call("orbit_fit_codebook_sphere", 2, 4, 0, 0.0, ctypes.byref(cb), None, None, None) == 1
    assert _call("orbit_fit_codebook_sphere", 64, 5, 0, 0.0, ctypes.byref(cb), None, None, None) == 1
    assert _call("orbit_fit_codebook_sphere", 64, 4, 0, 0.0, None, None, None, None) == 1
    with pytest.raises(ValueError):
        _lib().Codebook(64, 4, marginal="laplace")


def _call(name, *args):
    fn = getattr(_lib().lib, name)
    return fn(*args)


def _rot(d=256, h=64, perm=0x1000, signs=0x2000):
    return _lib()._RPBH(d, h, perm, signs)


P = ctypes.c_void_p
A16 = P(0x10000)        # a 16-byte aligned address that is never dereferenced
A8 = P(0x10008)


def test_fit_codebook_errors():
    cb = _lib()._Codebook()
    assert _call("orbit_fit_codebook", 256, 5, 0, 0.0, ctypes.byref(cb), None, None, None) == 1
    assert _call("orbit_fit_codebook", 256, 4, 0, 0.0, None, None, None, None) == 1
    assert _call("orbit_fit_codebook", 0, 4, 0, 0.0, ctypes.byref(cb), None, None, None) == 1


def test_quant_act_validation_before_any_hip_call():
    rbp = _lib()
    cb = rbp.Codebook(256, 4).struct
    idx, s = A16, A16
    ok = lambda rot, M=4, d=256, x=A16, dt=1, eps=1e-8, i=idx, o=s, dbg=None: _call(
        "orbit_quant_act", ctypes.byref(rot), ctypes.byref(cb), x, dt, M, d, eps, i, o, dbg, None)
    assert ok(_rot(), M=0) == 0                       # nothing to do, nothing enqueued
    assert ok(_rot(h=48)) == 2                        # h not a power of two
    assert ok(_rot(h=8)) == 2                         # h below 16
    assert ok(_rot(d=200, h=64), d=200) == 2          # d % h != 0
    assert ok(_rot(), d=512) == 2                     # rot->d != d
    assert ok(_rot(perm=0)) == 1                      # null perm
    assert ok(_rot(), dt=2) == 3                      # f16 input not accepted
    assert ok(_rot(), x=A8) == 1                      # misaligned input
    assert ok(_rot(), x=None) == 1
    assert ok(_rot(), eps=-1.0) == 1
    assert ok(_rot(), M=-1) == 2
    assert ok(_rot(d=32768, h=64), d=32768) == 2      # above the largest supported d
    bad = rbp.Codebook(256, 4).struct
    bad.thresholds[3] = bad.thresholds[5]             # unsorted
    assert _call("orbit_quant_act", ctypes.byref(_rot()), ctypes.byref(bad), A16, 1, 4, 256,
                 1e-8, A16, A16, None, None) == 1


def test_qlinear_validation():
    rbp = _lib()
    ca = rbp.Codebook(256, 4).struct
    c1 = rbp.Codebook(256, 1).struct
    call = lambda M=4, N=4, K=256, out_dt=1, a=A16, cw=ca, bias=None, bdt=0: _call(
        "orbit_qlinear", a, A16, ctypes.byref(ca), A16, A16, ctypes.byref(cw), bias, bdt,
        M, N, K, A16, out_dt, None)
    assert call(M=0) == 0 and call(N=0) == 0          # empty outputs: nothing to do
    assert call(K=192) == 2                           # K % 128 != 0
    assert call(K=0) == 2
    assert call(out_dt=2) == 3                        # fp16 output not offered
    assert call(a=A8) == 1                            # misaligned codes
    assert call(a=None) == 1
    assert call(cw=c1) == 4                           # 1-bit codes: no GEMM kernel
    assert call(bias=A16, bdt=2) == 3


def test_int8_validation():
    call = lambda group=128, K=256, xdt=2, M=4: _call(
        "orbit_int8_linear", A16, xdt, M, K, A16, A16, group, 4, None, 0, A16, 1, None)
    assert call(M=0) == 0
    assert call(group=64) == 4
    assert call(K=320) == 2
    assert call(xdt=1) == 3
    pack = lambda group=128, K=256: _call(
        "orbit_int8_pack_weights", ctypes.byref(_rot(d=K)), A16, 1, 4, K, group, A16, A16, None)
    assert pack(group=96) == 2 and pack(group=8) == 2 and pack(group=512) == 2


def test_status_strings():
    lib = _lib().lib
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"invalid shape"),
                       (3, b"unsupported dtype"), (4, b"unsupported configuration"),
                       (5, b"HIP error")]:
        assert lib.orbit_status_string(code) == text


@pytest.mark.parametrize("d,h,expect", [
    (3072, 128, 4096 + 3072 + 3072),   # butterfly section (at least 4 rounds) + matrix-core
                                       # words + scatter section (h = 128 / 256 packed-code rows)
    (1024, 64, 4096 + 1024),           # h = 64: no scatter section
    (12288, 256, 12288 + 12288 + 12288),
    (16384, 128, 16384 + 16384 + 16384),
    (5120, 128, 5120 + 5120),          # a row width the packed-code kernel does not take
    (512, 32, 4096),             # h = 32: no matrix-core kernel, no words
    (96, 16, 4096),              # d not a multiple of 512
    (2048, 512, 4096 + 2048),   # blocks of 512 .. 4096: the h = 128 order of words
    (3072, 100, 0),              # h not a power of two
    (100, 64, 0),                # d not a multiple of h
])
def test_gather_plan_length(d, h, expect):
    assert _lib().lib.orbit_rpbh_gather_len(d, h) == expect


def test_last_hip_error_reports_through_pointer():
    lib = _lib().lib
    assert lib.orbit_last_hip_error(None) == 1            # ORBIT_E_ARG
    code = ctypes.c_int(-1)
    assert lib.orbit_last_hip_error(ctypes.byref(code)) == 0
    assert code.value == 0                                # no failed HIP call on this thread


def test_build_gather_refuses_bad_arguments_before_any_hip_call():
    lib = _lib().lib
    assert lib.orbit_rpbh_build_gather(None, None, None) == 1
    rot = _rot(d=3072)
    rot.h = 100
    assert lib.orbit_rpbh_build_gather(ctypes.byref(rot), ctypes.c_void_p(16), None) == 2
