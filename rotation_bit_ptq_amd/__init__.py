"""Rotate-then-quantize linear layers on AMD MI355X (gfx950).

A thin ctypes binding of ``liborbit.so`` (C ABI in ``include/orbit.h``).
This module only marshals arguments: every step of the layer runs in the
library's HIP kernels on the caller's current torch stream.  Device buffers
are torch tensors; there is no CPU path, and importing fails if the library
has not been built (``__graft_entry__.build()`` or
``python rotation_bit_ptq_amd/build.py``).

Method (OrbitQuant paper page, Method): a randomized permuted block-Hadamard
rotation Pi = blkdiag(H_h D_i) P_pi is absorbed offline into the weights
(W' = W Pi^T, row norms in bf16, unit rows coded by a Lloyd-Max codebook) and
applied online to activations (x' = Pi x, split into ||x'|| and a coded unit
direction); the product of the two coded factors approximates W x with no
inverse rotation.  Also: the int8 per-group rotated weight-only path of the
int8 article (section 4) and its 4-bit sibling (int4 codes, two per byte).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "OrbitError", "Codebook", "Rotation", "fit_codebook", "pack_weights",
    "quant_act", "qlinear", "rotate", "int8_pack_weights", "int8_linear",
    "int4_pack_weights", "int4_linear",
    "packed_row_bytes", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liborbit.so")

F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
MAX_LEVELS = 256


class OrbitError(RuntimeError):
    pass


class _Codebook(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("d", ctypes.c_int32),
                ("centroids", ctypes.c_float * MAX_LEVELS),
                ("thresholds", ctypes.c_float * (MAX_LEVELS - 1))]


class _RPBH(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("h", ctypes.c_int32),
                ("perm", ctypes.c_void_p), ("sign_bits", ctypes.c_void_p),
                ("gather", ctypes.c_void_p), ("flags", ctypes.c_int32)]

RPBH_IDENTITY = 1  # set by the library's plan builder when perm is the identity (Block-RHT)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                         ctypes.c_float, ctypes.c_double)
    sig = {
        "orbit_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "orbit_last_hip_error": ([ctypes.c_void_p], ctypes.c_int),
        "orbit_fit_codebook": ([I32, I32, I32, D, P, P, P, P], ctypes.c_int),
        "orbit_fit_codebook_sphere": ([I32, I32, I32, D, P, P, P, P], ctypes.c_int),
        "orbit_rpbh_gather_len": ([I32, I32], I64),
        "orbit_rpbh_build_gather": ([P, P, P], ctypes.c_int),
        "orbit_pack_weights": ([P, P, P, ctypes.c_int, I64, I64, P, P, P], ctypes.c_int),
        "orbit_quant_act": ([P, P, P, ctypes.c_int, I64, I64, F, P, P, P, P], ctypes.c_int),
        "orbit_qlinear": ([P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, P,
                           ctypes.c_int, P], ctypes.c_int),
        "orbit_qlinear_act": ([P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, P,
                               ctypes.c_int, ctypes.c_int, P], ctypes.c_int),
        "orbit_rotate": ([P, P, ctypes.c_int, I64, I64, P, ctypes.c_int, P], ctypes.c_int),
        "orbit_int8_pack_weights": ([P, P, ctypes.c_int, I64, I64, I32, P, P, P], ctypes.c_int),
        "orbit_int4_pack_weights": ([P, P, ctypes.c_int, I64, I64, I32, P, P, P], ctypes.c_int),
        "orbit_int8_linear": ([P, ctypes.c_int, I64, I64, P, P, I32, I64, P, ctypes.c_int,
                               P, ctypes.c_int, P], ctypes.c_int),
        "orbit_int4_linear": ([P, ctypes.c_int, I64, I64, P, P, I32, I64, P, ctypes.c_int,
                               P, ctypes.c_int, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        try:
            fn = getattr(lib, name)
        except AttributeError as e:  # a library built from older sources
            raise ImportError(f"{LIB_PATH} lacks {name}; rebuild it with "
                              "__graft_entry__.build()") from e
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _check(status: int, what: str):
    if status != 0:
        msg = lib.orbit_status_string(status).decode()
        hip = ctypes.c_int(0)
        if status == 5:
            lib.orbit_last_hip_error(ctypes.byref(hip))
        raise OrbitError(f"{what}: {msg} (status {status}, hip {hip.value})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise OrbitError(f"{name} must be a torch tensor on a GPU")
    if not t.is_contiguous():
        raise OrbitError(f"{name} must be contiguous")
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def packed_row_bytes(d: int, bits: int) -> int:
    """Bytes of one packed row of d indices of `bits` bits."""
    return d * bits // 8


class Codebook:
    """A Lloyd-Max codebook in N(0,1) units (host memory).

    marginal="gauss": fitted to N(0,1), the large-d form of the rotated
    coordinate's marginal; "sphere": fitted to the exact marginal of one
    coordinate of a uniform direction on S^{d-1} (d >= 3)."""

    def __init__(self, d: int, bits: int, max_iter: int = 0, tol: float = 0.0,
                 marginal: str = "gauss"):
        fitters = {"gauss": "orbit_fit_codebook", "sphere": "orbit_fit_codebook_sphere"}
        if marginal not in fitters:
            raise ValueError(f"marginal must be one of {sorted(fitters)}")
        levels = 1 << bits
        self.struct = _Codebook()
        self.centroids_f64 = np.zeros(levels)
        self.thresholds_f64 = np.zeros(levels - 1)
        mse = ctypes.c_double(0.0)
        _check(getattr(lib, fitters[marginal])(
            d, bits, max_iter, tol, ctypes.byref(self.struct),
            self.centroids_f64.ctypes.data_as(ctypes.c_void_p),
            self.thresholds_f64.ctypes.data_as(ctypes.c_void_p), ctypes.byref(mse)),
            fitters[marginal])
        self.mse = mse.value
        self.bits, self.d, self.levels, self.marginal = bits, d, levels, marginal

    @property
    def centroids(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.struct.centroids)[: self.levels].copy()

    @property
    def thresholds(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.struct.thresholds)[: self.levels - 1].copy()


def fit_codebook(d: int, bits: int, marginal: str = "gauss") -> Codebook:
    return Codebook(d, bits, marginal=marginal)


class Rotation:
    """RPBH rotation parameters on a device: perm (gather order), sign bits, h,
    and (unless plan=False) the gather plan the row kernels read instead of
    deriving their offsets from perm and the signs.  Building the plan also
    lets the library set the identity-permutation flag (struct.flags)."""

    def __init__(self, perm, signs, h: int, device="cuda", plan: bool = True):
        perm = np.ascontiguousarray(perm, dtype=np.int32)
        signs = np.asarray(signs)
        d = perm.shape[0]
        bits = np.zeros((d + 31) // 32, dtype=np.uint32)
        neg = np.nonzero(signs < 0)[0]
        np.bitwise_or.at(bits, neg // 32, (np.uint32(1) << (neg % 32).astype(np.uint32)))
        self.d, self.h = d, int(h)
        self.perm = torch.from_numpy(perm).to(device)
        self.sign_bits = torch.from_numpy(bits.view(np.int32)).to(device)
        self.struct = _RPBH(d, int(h), self.perm.data_ptr(), self.sign_bits.data_ptr(), None, 0)
        self.gather = None
        n = lib.orbit_rpbh_gather_len(d, int(h)) if plan else 0
        if n > 0:
            self.gather = torch.empty((n,), dtype=torch.int16, device=self.perm.device)
            _check(lib.orbit_rpbh_build_gather(ctypes.byref(self.struct), _ptr(self.gather),
                                               _stream(self.perm.device)), "orbit_rpbh_build_gather")
            self.struct.gather = self.gather.data_ptr()


def pack_weights(rot: Rotation, cw: Codebook, W: torch.Tensor):
    """Offline: (packed indices uint8 [N, K*bits/8], row norms bf16 [N])."""
    _dev(W, "W")
    N, K = W.shape
    idx = torch.empty((N, packed_row_bytes(K, cw.bits)), dtype=torch.uint8, device=W.device)
    r = torch.empty((N,), dtype=torch.bfloat16, device=W.device)
    _check(lib.orbit_pack_weights(ctypes.byref(rot.struct), ctypes.byref(cw.struct), _ptr(W),
                                  _DT[W.dtype], N, K, _ptr(idx), _ptr(r), _stream(W.device)),
           "orbit_pack_weights")
    return idx, r


def quant_act(rot: Rotation, ca: Codebook, X: torch.Tensor, eps: float = 1e-8,
              debug_xrot: bool = False):
    """Online: (packed indices uint8 [M, K*bits/8], s float32 [M][, x' float32])."""
    _dev(X, "X")
    M, K = X.shape
    idx = torch.empty((M, packed_row_bytes(K, ca.bits)), dtype=torch.uint8, device=X.device)
    s = torch.empty((M,), dtype=torch.float32, device=X.device)
    xr = torch.empty((M, K), dtype=torch.float32, device=X.device) if debug_xrot else None
    _check(lib.orbit_quant_act(ctypes.byref(rot.struct), ctypes.byref(ca.struct), _ptr(X),
                               _DT[X.dtype], M, K, float(eps), _ptr(idx), _ptr(s), _ptr(xr),
                               _stream(X.device)), "orbit_quant_act")
    return (idx, s, xr) if debug_xrot else (idx, s)


ACTS = {None: 0, "gelu": 1}


def qlinear(idx_a, s, ca: Codebook, idx_w, r, cw: Codebook, K: int, bias=None,
            out_dtype=torch.bfloat16, out=None, act=None):
    """out[m, n] = act(s_m r_n / K * sum_k ca[ia] cw[iw] (+ bias)); act None or "gelu"."""
    for t, n in ((idx_a, "idx_a"), (s, "s"), (idx_w, "idx_w"), (r, "r")):
        _dev(t, n)
    if act not in ACTS:
        raise OrbitError(f"unknown activation {act!r}")
    M, N = idx_a.shape[0], idx_w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=idx_a.device)
    bias_dt = _DT[bias.dtype] if bias is not None else F32
    _check(lib.orbit_qlinear_act(_ptr(idx_a), _ptr(s), ctypes.byref(ca.struct), _ptr(idx_w),
                                 _ptr(r), ctypes.byref(cw.struct), _ptr(bias), bias_dt, M, N, K,
                                 _ptr(out), _DT[out.dtype], ACTS[act], _stream(idx_a.device)),
           "orbit_qlinear_act")
    return out


def rotate(rot: Rotation, X: torch.Tensor, out_dtype=torch.float16, out=None):
    """x' = Pi x per row."""
    _dev(X, "X")
    M, K = X.shape
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=X.device)
    _check(lib.orbit_rotate(ctypes.byref(rot.struct), _ptr(X), _DT[X.dtype], M, K, _ptr(out),
                            _DT[out.dtype], _stream(X.device)), "orbit_rotate")
    return out


def int8_pack_weights(rot: Rotation, W: torch.Tensor, group: int = 128):
    """Offline int8: (q int8 [N, K], scales fp16 [N, K/group])."""
    _dev(W, "W")
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    sc = torch.empty((N, K // group), dtype=torch.float16, device=W.device)
    _check(lib.orbit_int8_pack_weights(ctypes.byref(rot.struct), _ptr(W), _DT[W.dtype], N, K,
                                       group, _ptr(q), _ptr(sc), _stream(W.device)),
           "orbit_int8_pack_weights")
    return q, sc


def int8_linear(xrot: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, group: int = 128,
                bias=None, out_dtype=torch.bfloat16, out=None):
    """out = x' (q * scale)^T (+ bias), x' = Pi x in fp16."""
    for t, n in ((xrot, "xrot"), (q, "q"), (scale, "scale")):
        _dev(t, n)
    M, K = xrot.shape
    N = q.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=xrot.device)
    bias_dt = _DT[bias.dtype] if bias is not None else F32
    _check(lib.orbit_int8_linear(_ptr(xrot), _DT[xrot.dtype], M, K, _ptr(q), _ptr(scale), group,
                                 N, _ptr(bias), bias_dt, _ptr(out), _DT[out.dtype],
                                 _stream(xrot.device)), "orbit_int8_linear")
    return out


def int4_pack_weights(rot: Rotation, W: torch.Tensor, group: int = 128):
    """Offline int4: (q uint8 [N, K/2] two codes per byte, scales fp16 [N, K/group])."""
    _dev(W, "W")
    N, K = W.shape
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    sc = torch.empty((N, K // group), dtype=torch.float16, device=W.device)
    _check(lib.orbit_int4_pack_weights(ctypes.byref(rot.struct), _ptr(W), _DT[W.dtype], N, K,
                                       group, _ptr(q), _ptr(sc), _stream(W.device)),
           "orbit_int4_pack_weights")
    return q, sc


def int4_linear(xrot: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, group: int = 128,
                bias=None, out_dtype=torch.bfloat16, out=None):
    """out = x' (q * scale)^T (+ bias), x' = Pi x in fp16, q int4 two per byte."""
    for t, n in ((xrot, "xrot"), (q, "q"), (scale, "scale")):
        _dev(t, n)
    M, K = xrot.shape
    N = q.shape[0]
    if q.shape[1] * 2 != K:
        raise ValueError("q must be [N, K/2]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=xrot.device)
    bias_dt = _DT[bias.dtype] if bias is not None else F32
    _check(lib.orbit_int4_linear(_ptr(xrot), _DT[xrot.dtype], M, K, _ptr(q), _ptr(scale), group,
                                 N, _ptr(bias), bias_dt, _ptr(out), _DT[out.dtype],
                                 _stream(xrot.device)), "orbit_int4_linear")
    return out
