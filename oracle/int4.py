"""Int4 rotate-then-quantize weight-only path (fp64): the 4-bit sibling of
the int8 path in ``oracle/int8.py``.

OrbitQuant paper page (hyper.ai, "OrbitQuant"), section Experiments: the
ablations favour INT4 projections for the AdaLN layers; the page gives no
format for them.  Int8 rotated-weight article (cloud.baidu.com,
"量化旋转压缩主模型技术解析", section 4 "How it works"): rotate -> per-group
scale -> round -> store (q, scale, rotation metadata); at load time
dequantize -> inverse rotate -> ordinary layer forward.

Readings taken (none of this is fixed by the pages): the int8 recipe with
the symmetric 4-bit range, i.e. W' = W Pi^T with the RPBH rotation, groups
of g consecutive columns of W', scale = fp16(max|w'| / 7),
q = clamp(round_half_even(w' / scale), -7, 7), q = 0 when scale = 0; codes
stored as two's-complement nibbles, two per byte, element 2j in the low
nibble of byte j (the LSB-first stream of the 4-bit codebook indices).
"""
import numpy as np

from .numfmt import f64_to_f16_bits, f16_bits_to_f64, f64_to_f32
from .rotation import rpbh_rotate, rpbh_inverse_rotate

QMAX = 7


def int4_pack(W, perm, signs, h, group=128, decision="f32"):
    """Returns dict(q int8 [N, d] in [-7, 7], scale_f16 uint16 [N, d/group], wrot).

    decision="f32": amax, amax / 7 and w' / scale are float32 operations on
    float32(w'), and the scale is rounded to fp16 from that float32 value;
    decision="f64" does the same in float64.
    """
    W = np.asarray(W, dtype=np.float64)
    N, d = W.shape
    if d % group:
        raise ValueError("d must be a multiple of the group size")
    wrot = rpbh_rotate(W, perm, signs, h)
    groups = wrot.reshape(N, d // group, group)
    if decision == "f32":
        g = f64_to_f32(groups)
        amax = np.max(np.abs(g), axis=-1)
        scale_bits = f64_to_f16_bits((amax / np.float32(QMAX)).astype(np.float64))
        sc = f16_bits_to_f64(scale_bits).astype(np.float32)
    elif decision == "f64":
        g = groups
        amax = np.max(np.abs(g), axis=-1)
        scale_bits = f64_to_f16_bits(amax / float(QMAX))
        sc = f16_bits_to_f64(scale_bits)
    else:
        raise ValueError("decision must be 'f32' or 'f64'")
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(sc[..., None] > 0, g / sc[..., None], 0.0)
    q = np.clip(np.rint(ratio), -QMAX, QMAX)
    return dict(q=q.reshape(N, d).astype(np.int8), scale_f16=scale_bits, wrot=wrot)


def pack_nibbles(q):
    """int8 codes [N, d] (d even) -> uint8 [N, d/2]; code 2j goes to the low
    nibble of byte j, code 2j+1 to the high nibble, both two's complement."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, d):
    """uint8 [N, d/2] -> int8 codes [N, d] (sign-extended nibbles)."""
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty((p.shape[0], d), dtype=np.int64)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def int4_dequant(q, scale_f16, group=128):
    """W^' = q * scale per (row, group), in float64."""
    q = np.asarray(q, dtype=np.float64)
    N, d = q.shape
    sc = f16_bits_to_f64(scale_f16)
    return (q.reshape(N, d // group, group) * sc[..., None]).reshape(N, d)


def int4_linear(X, q, scale_f16, perm, signs, h, group=128):
    """Load-and-run: W^ = inverse_rotate(dequant(q, scale)); y = X W^^T."""
    W_hat = rpbh_inverse_rotate(int4_dequant(q, scale_f16, group), perm, signs, h)
    return np.asarray(X, dtype=np.float64) @ W_hat.T, W_hat


def int4_linear_rotated(Xrot, q, scale_f16, group=128):
    """The equal form the kernels use: (X Pi^T) W^'^T, no inverse rotation."""
    return np.asarray(Xrot, dtype=np.float64) @ int4_dequant(q, scale_f16, group).T
