"""Seeded synthetic workloads for the rotate-then-quantize linear layer.

This module only draws random numbers and stores them in the input formats
the layer reads (fp32, or bf16 as raw uint16 bit patterns).  It holds none of
the method's arithmetic: no rotation, no norm, no codebook, no quantization.
Both the fp64 oracle and the HIP library receive the arrays made here, and
nothing else is shared between them.

The random rotation parameters of the RPBH transform (the permutation pi and
the Rademacher signs D) are random draws of the method; they are drawn here
and passed as inputs to both sides.

Workloads (diffusion-transformer shaped; the pages measure on trained image
and video DiTs, which these synthetic tensors stand in for):

  1 tiny_w4a4   d_in=d_out=256, h=64, 64 fp32 tokens ~N(0,1) with 4 outlier
                channels x30; W fp32 ~N(0, 0.02^2); 16-level codebooks.
  2 image_w4a4  d=3072, h=128, 4096 bf16 tokens ~N(0,1), 15 channels (0.5 %)
                x50, per-token scale exp(N(0, 0.5^2)); W ~N(0, 1/3072) bf16.
  3 int8_w8     W 4096x4096 bf16 ~ Student-t(4) * 0.02; h=128, group 128;
                16384 bf16 tokens ~N(0,1).
  4 mlp_w2a4    up 3072->12288 then down 12288->3072, h=256, 16384 tokens with
                the image activation recipe; W_up ~N(0,1/3072),
                W_down ~N(0,1/12288); 4-level weight, 16-level act codebooks.
  5 video_w4a6  d_in=2048, d_out=8192, h=128, 32768 tokens = 8 frames x 4096;
                ~N(0,1) with 20 channels (1 %) x40 plus a per-frame drift
                ~N(0, 0.3 I); 64-level act, 16-level weight codebooks.

Every tensor is drawn in float32 from numpy's PCG64, then rounded to
nearest-even into its storage type.  Seeds: ``SeedSequence(1000 + config)``,
spawned into named child streams, so a smaller token or row count draws the
leading rows of the full-size tensor (prefix-consistent).
"""
from __future__ import annotations

import numpy as np

__all__ = ["CONFIGS", "make", "f32_to_bf16_bits", "bf16_bits_to_f32"]

# Child stream order of SeedSequence(1000 + config).spawn(len(_STREAMS)).
_STREAMS = ("perm", "signs", "W", "X", "outlier", "extra",
            "perm2", "signs2", "W2")

CONFIGS = {
    1: dict(name="tiny_w4a4", M=64, K=256, N=256, h=64, bits_a=4, bits_w=4,
            x_dtype="f32", w_dtype="f32", out_dtype="f32"),
    2: dict(name="image_w4a4", M=4096, K=3072, N=3072, h=128, bits_a=4,
            bits_w=4, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16"),
    3: dict(name="int8_w8", M=16384, K=4096, N=4096, h=128, group=128,
            x_dtype="bf16", w_dtype="bf16", out_dtype="bf16"),
    4: dict(name="mlp_w2a4", M=16384, K=3072, N=12288, h=256, bits_a=4,
            bits_w=2, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16"),
    5: dict(name="video_w4a6", M=32768, K=2048, N=8192, h=128, bits_a=6,
            bits_w=4, x_dtype="bf16", w_dtype="bf16", out_dtype="bf16",
            frame_tokens=4096),
}

EPS = 1e-8  # the epsilon added to the activation norm (s + eps)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(config: int):
    ss = np.random.SeedSequence(1000 + config)
    kids = ss.spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(k))
            for name, k in zip(_STREAMS, kids)}


def _rotation(gp, gs, d):
    perm = gp.permutation(d).astype(np.int32)
    signs = np.where(gs.integers(0, 2, size=d) == 1, -1, 1).astype(np.int8)
    return perm, signs


def _outlier_acts(gx, go, M, K, n_out, factor, lognormal_sigma=None,
                  drift=None, frame_tokens=None, ge=None):
    """Gaussian tokens with a few boosted channels (DiT activation outliers)."""
    X = gx.standard_normal((M, K), dtype=np.float32)
    ch = go.choice(K, size=n_out, replace=False)
    X[:, ch] *= np.float32(factor)
    if lognormal_sigma is not None:
        X *= np.exp(ge.standard_normal(M, dtype=np.float32)
                    * np.float32(lognormal_sigma))[:, None]
    if drift is not None:
        n_frames = (M + frame_tokens - 1) // frame_tokens
        off = ge.standard_normal((n_frames, K), dtype=np.float32) * np.float32(np.sqrt(drift))
        X += np.repeat(off, frame_tokens, axis=0)[:M]
    return X


def make(config: int, M: int | None = None, N: int | None = None,
         K: int | None = None, h: int | None = None) -> dict:
    """Draw the inputs of a workload.  Optional overrides shrink a dimension.

    Returns a dict with the workload metadata and arrays:
      perm int32[K], signs int8[K] (+1/-1),
      X  [M, K] float32 or bf16 bits (uint16),
      W  [N, K] float32 or bf16 bits (uint16),
    and for the MLP pair also perm2, signs2 [N], W2 [K, N] (the down layer).
    """
    cfg = dict(CONFIGS[config])
    M = cfg["M"] if M is None else M
    N = cfg["N"] if N is None else N
    K = cfg["K"] if K is None else K
    h = cfg["h"] if h is None else h
    cfg.update(M=M, N=N, K=K, h=h, config=config, eps=EPS)
    g = _streams(config)
    perm, signs = _rotation(g["perm"], g["signs"], K)
    out = dict(cfg, perm=perm, signs=signs)

    if config == 1:
        W = g["W"].standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        X = _outlier_acts(g["X"], g["outlier"], M, K, 4, 30.0)
        out.update(W=W, X=X)
    elif config == 2:
        W = g["W"].standard_normal((N, K), dtype=np.float32) * np.float32(1 / np.sqrt(K))
        X = _outlier_acts(g["X"], g["outlier"], M, K, int(round(0.005 * K)), 50.0,
                          lognormal_sigma=0.5, ge=g["extra"])
        out.update(W=f32_to_bf16_bits(W), X=f32_to_bf16_bits(X))
    elif config == 3:
        W = (g["W"].standard_t(4, size=(N, K)) * 0.02).astype(np.float32)
        X = g["X"].standard_normal((M, K), dtype=np.float32)
        out.update(W=f32_to_bf16_bits(W), X=f32_to_bf16_bits(X))
    elif config == 4:
        W = g["W"].standard_normal((N, K), dtype=np.float32) * np.float32(1 / np.sqrt(K))
        X = _outlier_acts(g["X"], g["outlier"], M, K, int(round(0.005 * K)), 50.0,
                          lognormal_sigma=0.5, ge=g["extra"])
        perm2, signs2 = _rotation(g["perm2"], g["signs2"], N)
        W2 = g["W2"].standard_normal((K, N), dtype=np.float32) * np.float32(1 / np.sqrt(N))
        out.update(W=f32_to_bf16_bits(W), X=f32_to_bf16_bits(X), perm2=perm2,
                   signs2=signs2, W2=f32_to_bf16_bits(W2), bits_w2=2, bits_a2=4)
    elif config == 5:
        W = g["W"].standard_normal((N, K), dtype=np.float32) * np.float32(1 / np.sqrt(K))
        X = _outlier_acts(g["X"], g["outlier"], M, K, int(round(0.01 * K)), 40.0,
                          drift=0.3, frame_tokens=cfg["frame_tokens"], ge=g["extra"])
        out.update(W=f32_to_bf16_bits(W), X=f32_to_bf16_bits(X))
    else:
        raise ValueError(f"unknown workload {config}")
    return out


def rotation_params(d: int, seed: int):
    """A standalone seeded (perm, signs) pair for dimension d."""
    ss = np.random.SeedSequence(seed).spawn(2)
    return _rotation(np.random.Generator(np.random.PCG64(ss[0])),
                     np.random.Generator(np.random.PCG64(ss[1])), d)
