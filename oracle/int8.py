"""Int8 rotate-then-quantize weight-only path (fp64), literally as written.

Int8 rotated-weight article (cloud.baidu.com, "量化旋转压缩主模型技术解析",
section 4 "How it works"): pack = orthogonal rotation -> per-group scale ->
round(rotated / scale) -> store (q, scale, rotation metadata); load-and-run =
dequantize -> inverse rotation -> ordinary layer forward.

Readings taken: the rotation is the RPBH rotation of the OrbitQuant page
applied as W' = W Pi^T (rows rotated, groups run along the input dimension);
groups of g consecutive columns of W'; scale = fp16(max|w'| / 127);
q = clamp(round_half_even(w' / scale), -127, 127), q = 0 when scale = 0
(the symmetric [-127, 127] range of the workload, not the [-128, 127] that the
first article mentions).
"""
import numpy as np

from .numfmt import f64_to_f16_bits, f16_bits_to_f64, f64_to_f32
from .rotation import rpbh_rotate, rpbh_inverse_rotate


def int8_pack(W, perm, signs, h, group=128, decision="f32"):
    """Returns dict(q int8 [N, d], scale_f16 uint16 [N, d/group], wrot).

    decision="f32": the scale and the codes are decided in float32 from
    float32(w'): amax, amax/127 and w'/scale are float32 operations, the
    scale is rounded to fp16 from that float32 value.  decision="f64" does
    the same in float64.
    """
    W = np.asarray(W, dtype=np.float64)
    N, d = W.shape
    if d % group:
        raise ValueError("d must be a multiple of the group size")
    wrot = rpbh_rotate(W, perm, signs, h)
    G = wrot.reshape(N, d // group, group)
    if decision == "f32":
        G32 = f64_to_f32(G)
        amax = np.max(np.abs(G32), axis=-1)
        scale_bits = f64_to_f16_bits((amax / np.float32(127.0)).astype(np.float64))
        sc = f16_bits_to_f64(scale_bits).astype(np.float32)
        with np.errstate(invalid="ignore", divide="ignore"):
            ratio = G32 / sc[..., None]
        ratio = np.where(sc[..., None] > 0, ratio, np.float32(0.0))
        q = np.clip(np.rint(ratio), -127, 127)
    elif decision == "f64":
        amax = np.max(np.abs(G), axis=-1)
        scale_bits = f64_to_f16_bits(amax / 127.0)
        sc = f16_bits_to_f64(scale_bits)
        with np.errstate(invalid="ignore", divide="ignore"):
            ratio = np.where(sc[..., None] > 0, G / sc[..., None], 0.0)
        q = np.clip(np.rint(ratio), -127, 127)
    else:
        raise ValueError("decision must be 'f32' or 'f64'")
    return dict(q=q.reshape(N, d).astype(np.int8), scale_f16=scale_bits, wrot=wrot)


def int8_dequant(q, scale_f16, group=128):
    """W^' = q * scale, per (row, group), in float64."""
    q = np.asarray(q, dtype=np.float64)
    N, d = q.shape
    sc = f16_bits_to_f64(scale_f16)
    return (q.reshape(N, d // group, group) * sc[..., None]).reshape(N, d)


def int8_linear(X, q, scale_f16, perm, signs, h, group=128):
    """Load-and-run: W^ = inverse_rotate(dequant(q, scale)); y = X W^^T."""
    Wq_rot = int8_dequant(q, scale_f16, group)
    W_hat = rpbh_inverse_rotate(Wq_rot, perm, signs, h)    # W^ = W^' Pi
    return np.asarray(X, dtype=np.float64) @ W_hat.T, W_hat


def int8_linear_rotated(Xrot, q, scale_f16, group=128):
    """The equal form the kernels use: (X Pi^T) W^'^T (no inverse rotation)."""
    return np.asarray(Xrot, dtype=np.float64) @ int8_dequant(q, scale_f16, group).T
