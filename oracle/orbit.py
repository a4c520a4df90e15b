"""The OrbitQuant linear layer, step by step in fp64.

OrbitQuant page, Method:
  offline  W' = W Pi_d^T; each row w'_i = r'_i * w~'_i with r'_i = ||w'_i||_2
           (stored in BF16) and w~'_i quantized by the Lloyd-Max codebook;
           W^' = diag(r') Q_bw(W~').
  online   x' = Pi_d x; s = ||x'||_2; x~' = x' / (s + eps);
           x^' = s Q_ba(x~').
  product  W^' x^' ~ W x: the rotation cancels, nothing is inverse-rotated
           at run time.

Codebooks are in N(0,1) units (see codebook.py): a unit direction v is
quantized through u = sqrt(d) v, index idx = #{j : t_j < u}, and decodes to
c_idx / sqrt(d).  So <Q(w~), Q(x~)> = (1/d) sum_k c_w[iw_k] c_a[ia_k] and the
layer output is  y[m, n] = r^_n s_m (1/d) sum_k c_a[ia[m,k]] c_w[iw[n,k]].

Readings taken (the pages are silent): eps is an argument, weights use no eps
and a zero row quantizes to index #{t_j < 0} with r = 0 so it contributes 0;
no bias unless given; the quantizer is the nearest-centroid rule written as a
threshold count.
"""
import numpy as np
from scipy.special import erf

from .numfmt import f64_to_bf16_bits, bf16_bits_to_f64, f64_to_f32
from .rotation import rpbh_rotate


def quantize_codes(u, thresholds, decision="f32"):
    """idx = #{j : t_j < u} for every element of u (N(0,1) units).

    decision="f32": the comparison is made between float32(u) and
    float32(t_j), the precision the kernels decide in.  decision="f64"
    compares the float64 values.
    """
    u = np.asarray(u, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    if decision == "f32":
        u, t = f64_to_f32(u), f64_to_f32(t)
    elif decision != "f64":
        raise ValueError("decision must be 'f32' or 'f64'")
    idx = np.zeros(u.shape, dtype=np.int64)
    for tj in t:                      # count thresholds strictly below u
        idx += (tj < u)
    return idx.astype(np.uint8)


def boundary_band(u, thresholds, band=1e-6):
    """True where |u - t_j| <= band for some threshold (fp64 values)."""
    u = np.asarray(u, dtype=np.float64)
    near = np.zeros(u.shape, dtype=bool)
    for tj in np.asarray(thresholds, dtype=np.float64):
        near |= np.abs(u - tj) <= band
    return near


def pack_indices(idx, bits):
    """Pack each row of b-bit indices into an LSB-first byte stream.

    Index k of a row occupies bits [k*b, (k+1)*b) of the stream, and bit n of
    the stream is bit (n mod 8) of byte n // 8.  Rows must hold a whole
    number of bytes (k*b divisible by 8).
    """
    idx = np.asarray(idx, dtype=np.int64)
    *lead, n = idx.shape
    if (n * bits) % 8:
        raise ValueError("row length * bits must be a multiple of 8")
    if idx.size and (idx.min() < 0 or idx.max() >= (1 << bits)):
        raise ValueError("index out of range for the bit width")
    stream = np.zeros((*lead, n * bits), dtype=np.uint8)
    for b in range(bits):
        stream[..., b::bits] = (idx >> b) & 1
    stream = stream.reshape(*lead, n * bits // 8, 8)
    weights = (1 << np.arange(8)).astype(np.int64)
    return (stream * weights).sum(axis=-1).astype(np.uint8)


def unpack_indices(packed, bits, n):
    """Inverse of pack_indices: the first n b-bit indices of every row."""
    packed = np.asarray(packed, dtype=np.uint8)
    *lead, nbytes = packed.shape
    stream = ((packed[..., :, None] >> np.arange(8)) & 1).reshape(*lead, nbytes * 8)
    stream = stream[..., : n * bits].reshape(*lead, n, bits).astype(np.int64)
    return (stream << np.arange(bits)).sum(axis=-1).astype(np.uint8)


def pack_weights(W, perm, signs, h, cb, bits, decision="f32"):
    """Offline weight path: W' = W Pi^T, r' = ||w'_i||, quantize w'_i / r'_i.

    W [N, d] (float64 values).  Returns dict with
      idx [N, d] uint8, packed [N, d*bits/8] uint8, r (fp64 norms),
      r_bf16 (uint16 bits: the stored norms), u (fp64 N(0,1)-unit values),
      wrot (W' rows).
    """
    W = np.asarray(W, dtype=np.float64)
    d = W.shape[-1]
    wrot = rpbh_rotate(W, perm, signs, h)                 # rows: Pi w_i
    r = np.sqrt(np.sum(wrot * wrot, axis=-1))
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.where(r[:, None] > 0, np.sqrt(d) * wrot / r[:, None], 0.0)
    idx = quantize_codes(u, cb["thresholds"], decision)
    r_store = f64_to_bf16_bits(f64_to_f32(r) if decision == "f32" else r)
    return dict(idx=idx, packed=pack_indices(idx, bits), r=r, r_bf16=r_store,
                u=u, wrot=wrot)


def quant_act(X, perm, signs, h, cb, bits, eps, decision="f32"):
    """Online activation path: x' = Pi x, s = ||x'||, u = sqrt(d) x'/(s + eps).

    X [M, d].  Returns dict with idx, packed, s (fp64), xrot (x'), u.
    """
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[-1]
    xrot = rpbh_rotate(X, perm, signs, h)
    s = np.sqrt(np.sum(xrot * xrot, axis=-1))
    u = np.sqrt(d) * xrot / (s[:, None] + eps)
    idx = quantize_codes(u, cb["thresholds"], decision)
    return dict(idx=idx, packed=pack_indices(idx, bits), s=s, xrot=xrot, u=u)


def qlinear_codes(idx_a, s, cent_a, idx_w, r_bf16, cent_w, d, bias=None):
    """y[m, n] = r^_n s_m (1/d) sum_k c_a[ia[m,k]] c_w[iw[n,k]] (+ bias[n]).

    Takes unpacked indices; r_bf16 are the stored bf16 norms (bits).  This is
    the "same codes" product: given the codes, the output is fixed.
    """
    A = np.asarray(cent_a, dtype=np.float64)[np.asarray(idx_a, dtype=np.int64)]
    B = np.asarray(cent_w, dtype=np.float64)[np.asarray(idx_w, dtype=np.int64)]
    r = bf16_bits_to_f64(r_bf16)
    y = (A @ B.T) * (np.asarray(s, dtype=np.float64)[:, None] * r[None, :] / d)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def qlinear_unquantized(X, W, perm, signs, h, eps=0.0):
    """The same factorisation with the quantizer removed (Q = identity):
    r'_n s_m <w~'_n, x~'_m>, which equals (W x)_m,n exactly when eps = 0."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    xr = rpbh_rotate(X, perm, signs, h)
    wr = rpbh_rotate(W, perm, signs, h)
    s = np.sqrt(np.sum(xr * xr, axis=-1))
    r = np.sqrt(np.sum(wr * wr, axis=-1))
    xt = xr / (s[:, None] + eps)
    wt = wr / r[:, None]
    return (xt @ wt.T) * s[:, None] * r[None, :]


def gelu_erf(x):
    """GELU with the exact erf form: x * (1 + erf(x / sqrt 2)) / 2."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
