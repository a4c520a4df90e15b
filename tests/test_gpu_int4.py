"""GPU parity of the int4 rotated weight-only path against the oracle.

The 4-bit sibling of the int8 path (int8 article, section 4; INT4
projections of the OrbitQuant page's Experiments section): the packer
rotates, takes a per-group fp16 scale max|w'|/7 and rounds to [-7, 7]; the
GPU runs the equal form (X Pi^T)(q * scale)^T, the oracle the literal
dequant -> inverse rotate -> X W^T in fp64.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import int4
from parity import OUT_TOL, as_f64, bits_of, check_group_codes, out_f64, rel_fro, to_dev

pytestmark = pytest.mark.gpu

# On the GPU's own fp16 x' the kernel differs from the exact product only by
# rounding each decoded weight q * scale to fp16 (relative error <= 2^-11,
# unbiased) and fp32 accumulation, so the relative Frobenius error of the
# output stays below 2^-11.
SAME_X_TOL = 2.0 ** -11


def _check_pack(q_dev, sc_dev, W, perm, signs, h, group=128):
    wrot = oracle.rpbh_rotate(W, perm, signs, h)
    packed = q_dev.cpu().numpy()
    q = int4.unpack_nibbles(packed, W.shape[1])
    check_group_codes(q, bits_of(sc_dev), wrot, group, int4.QMAX, f"int4-K{W.shape[1]}-h{h}")
    # the bytes themselves: two's-complement nibbles, code 2j in the low nibble
    assert np.array_equal(packed, int4.pack_nibbles(q))
    return q


@pytest.mark.parametrize("K,h,f32", [
    (4096, 128, False),   # bf16 rows, transposed-gather kernel
    (1024, 64, False),
    (2048, 256, False),
    (512, 32, False),     # bf16 rows, consecutive kernel
    (1024, 128, True),    # fp32 rows
    (8192, 128, False),   # long rows: one workgroup per row
])
def test_int4_pack_matches_oracle(gpu_lib, K, h, f32):
    rbp = gpu_lib
    inp = synth.make(3, M=8, N=300, K=K, h=h)
    W = to_dev(inp["W"])
    if f32:
        W = W.float()
    rot = rbp.Rotation(inp["perm"], inp["signs"], h)
    q, sc = rbp.int4_pack_weights(rot, W, 128)
    torch.cuda.synchronize()
    assert q.shape == (300, K // 2)
    _check_pack(q, sc, as_f64(inp["W"]), inp["perm"], inp["signs"], h)


def test_int4_pack_zero_rows_and_groups(gpu_lib):
    rbp = gpu_lib
    K = 1024
    perm, signs = synth.rotation_params(K, 5)
    W = np.zeros((4, K), np.float32)
    W[1] = np.random.default_rng(1).standard_normal(K)
    rot = rbp.Rotation(perm, signs, 128)
    q, sc = rbp.int4_pack_weights(rot, torch.from_numpy(W).cuda(), 128)
    torch.cuda.synchronize()
    assert torch.all(q[0] == 0) and torch.all(q[2:] == 0)
    assert np.all(bits_of(sc)[[0, 2, 3]] == 0)
    _check_pack(q, sc, W.astype(np.float64), perm, signs, 128)


def test_int4_linear_matches_literal_oracle(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(3, M=300, N=200)
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    q, sc = rbp.int4_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    out = rbp.int4_linear(xr, q, sc, 128)
    qi = int4.unpack_nibbles(q.cpu().numpy(), xr.shape[1])
    y, _ = int4.int4_linear(as_f64(inp["X"]), qi, bits_of(sc), inp["perm"], inp["signs"],
                            inp["h"], 128)
    assert rel_fro(out_f64(out), y) < OUT_TOL
    out32 = rbp.int4_linear(xr, q, sc, 128, out_dtype=torch.float32)
    assert rel_fro(out_f64(out32), y) < 1e-3
    y_same = int4.int4_linear_rotated(oracle.f16_bits_to_f64(bits_of(xr)), qi, bits_of(sc))
    assert rel_fro(out_f64(out32), y_same) < SAME_X_TOL


@pytest.mark.parametrize("M,N,K", [(1, 7, 128), (33, 129, 256), (257, 300, 1024),
                                   (1024, 512, 3072)])
def test_int4_linear_ragged(gpu_lib, M, N, K):
    rbp = gpu_lib
    inp = synth.make(3, M=M, N=N, K=K, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int4_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    bias = torch.from_numpy(np.random.default_rng(2).standard_normal(N).astype(np.float32)).cuda()
    out = rbp.int4_linear(xr, q, sc, 128, bias=bias, out_dtype=torch.float32)
    qi = int4.unpack_nibbles(q.cpu().numpy(), K)
    y = int4.int4_linear_rotated(oracle.f16_bits_to_f64(bits_of(xr)), qi, bits_of(sc))
    assert rel_fro(out_f64(out), y + bias.cpu().numpy()) < SAME_X_TOL


def test_int4_rejects_bad_shapes(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(3, M=4, N=8, K=256, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int4_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    with pytest.raises(rbp.OrbitError):
        rbp.int4_linear(xr, q, sc, 64)                # group must be 128
    with pytest.raises(ValueError):
        rbp.int4_linear(xr, q[:, :64].contiguous(), sc, 128)


# Products with at least 128 tiles of 256 x 256 take the LDS-staged kernel;
# (4096, 2049, 384) has an odd number of scale entries and takes the
# register-fed kernel instead.
STAGED = [(4096, 2048, 512), (4000, 2100, 256), (4096, 2048, 128), (4096, 2049, 384),
          (4096, 2048, 4096),   # the int8 workload's K
          # narrow batches (up to 32 tokens: one workgroup per 32 weight rows; 64:
          # small tiles)
          (24, 600, 3072), (64, 1000, 1024), (5, 33, 128),
          # up to 16 tokens and 8, 16, 24 or 32 groups per row: one workgroup per
          # compute unit walking 16-row slabs (the AdaLN-style projection at full
          # size; a single slab; more than 2048 slabs, eight per workgroup)
          (16, 18432, 3072), (16, 4608, 3072), (1, 100, 1024), (7, 1000, 2048),
          (16, 4100, 4096), (12, 16, 3072), (3, 40000, 1024)]


@pytest.mark.parametrize("M,N,K", STAGED)
def test_int4_linear_staged_tiles(gpu_lib, M, N, K):
    rbp = gpu_lib
    inp = synth.make(3, M=M, N=N, K=K, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int4_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    bias = torch.from_numpy(np.random.default_rng(3).standard_normal(N).astype(np.float32)).cuda()
    qi = int4.unpack_nibbles(q.cpu().numpy(), K)
    x16 = oracle.f16_bits_to_f64(bits_of(xr))
    y = int4.int4_linear_rotated(x16, qi, bits_of(sc)) + bias.cpu().numpy()
    out32 = rbp.int4_linear(xr, q, sc, 128, bias=bias, out_dtype=torch.float32)
    assert rel_fro(out_f64(out32), y) < SAME_X_TOL
    out16 = rbp.int4_linear(xr, q, sc, 128, bias=bias)
    assert rel_fro(out_f64(out16), y) < OUT_TOL


def test_int4_workload_full_size_sampled(gpu_lib):
    """The int8 workload's shape with 4-bit codes (16384 tokens, 4096 -> 4096,
    h = 128), sampled outputs against the literal oracle."""
    rbp = gpu_lib
    inp = synth.make(3)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int4_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    out = rbp.int4_linear(xr, q, sc, 128)
    g = np.random.default_rng(9)
    ms = np.sort(g.choice(inp["M"], 64, replace=False))
    ns = np.sort(g.choice(inp["N"], 96, replace=False))
    qi = int4.unpack_nibbles(q[ns].cpu().numpy(), inp["K"])
    y, _ = int4.int4_linear(as_f64(inp["X"][ms]), qi, bits_of(sc[ns]), inp["perm"],
                            inp["signs"], 128)
    assert rel_fro(out_f64(out[ms][:, ns]), y) < OUT_TOL
