"""GPU parity of the int8 rotated weight-only path against the oracle.

Int8 article (section 4): the packer rotates, takes a per-group scale and
rounds; load-and-run dequantizes, inverse-rotates and runs the layer.  The
GPU computes the equal form (X Pi^T)(q * scale)^T; the oracle runs the
literal dequant -> inverse rotate -> X W^T in fp64.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import OUT_TOL, as_f64, bits_of, check_group_codes, out_f64, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _setup(rbp, M=300, N=256):
    inp = synth.make(3, M=M, N=N)
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    return inp, rot


def test_rotate_f16_and_f32(gpu_lib):
    rbp = gpu_lib
    inp, rot = _setup(rbp)
    ref = oracle.rpbh_rotate(as_f64(inp["X"]), inp["perm"], inp["signs"], inp["h"])
    x32 = rbp.rotate(rot, to_dev(inp["X"]), torch.float32).cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(x32 - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() <= 1e-5
    x16 = oracle.f16_bits_to_f64(bits_of(rbp.rotate(rot, to_dev(inp["X"]), torch.float16)))
    ref16 = oracle.f16_bits_to_f64(oracle.f64_to_f16_bits(ref))
    diff = x16 != ref16
    # off rounding ties the fp16 value is the nearest one to the exact x'; the
    # fp32 butterflies carry an absolute error of ~1e-7 of the token's scale,
    # so a tie is "near" within 1e-6 of the token's largest coordinate
    if diff.any():
        scale = np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
        ulp = np.spacing(np.abs(ref16[diff]).astype(np.float16)).astype(np.float64)
        dist_to_tie = np.abs(np.abs(ref[diff] - ref16[diff]) - ulp / 2)
        assert np.all(dist_to_tie <= 1e-6 * scale[diff])
        assert np.all(np.abs(x16[diff] - ref16[diff]) <= ulp * 1.0001)
    assert diff.mean() < 1e-4


def _check_f16_rotation(x16, ref):
    ref16 = oracle.f16_bits_to_f64(oracle.f64_to_f16_bits(ref))
    diff = x16 != ref16
    if diff.any():  # only at fp16 rounding ties, as above
        scale = np.abs(ref).max(axis=1, keepdims=True) * np.ones_like(ref)
        ulp = np.spacing(np.abs(ref16[diff]).astype(np.float16)).astype(np.float64)
        dist_to_tie = np.abs(np.abs(ref[diff] - ref16[diff]) - ulp / 2)
        assert np.all(dist_to_tie <= 1e-6 * scale[diff])
        assert np.all(np.abs(x16[diff] - ref16[diff]) <= ulp * 1.0001)
    assert diff.mean() < 1e-4


# fp16 rotations of bf16 rows with h = 64, 128, 256 and d = 1024 .. 4096 run
# the Hadamard on the matrix cores; 93 rows, one of them zero
@pytest.mark.parametrize("d,h,ident", [(1024, 64, False), (2048, 256, False), (3072, 128, False),
                                        (4096, 64, False), (3072, 256, False), (2048, 128, True)])
def test_rotate_f16_matrix_core_shapes(gpu_lib, d, h, ident):
    # ident: Block-RHT (pi = identity)
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, 3 * d + h)
    if ident:
        perm = np.arange(d, dtype=np.int32)
    g = np.random.default_rng(d - h)
    X = synth.f32_to_bf16_bits(g.standard_normal((93, d)).astype(np.float32))
    X[40] = 0
    rot = rbp.Rotation(perm, signs, h)
    ref = oracle.rpbh_rotate(as_f64(X), perm, signs, h)
    x16 = oracle.f16_bits_to_f64(bits_of(rbp.rotate(rot, to_dev(X), torch.float16)))
    assert np.all(x16[40] == 0)
    _check_f16_rotation(x16, ref)


@pytest.mark.parametrize("N", [300, 4096])
def test_int8_pack_matches_oracle(gpu_lib, N):
    # N = 4096: the full 4096 x 4096 weight of the int8 workload
    rbp = gpu_lib
    inp, rot = _setup(rbp, M=8, N=N)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    wrot = oracle.rpbh_rotate(as_f64(inp["W"]), inp["perm"], inp["signs"], inp["h"])
    check_group_codes(q.cpu().numpy(), bits_of(sc), wrot, 128, 127, f"int8-pack-N{N}")


def test_int8_linear_matches_literal_oracle(gpu_lib):
    rbp = gpu_lib
    inp, rot = _setup(rbp, M=300, N=200)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    out = rbp.int8_linear(xr, q, sc, 128)
    y, _ = oracle.int8_linear(as_f64(inp["X"]), q.cpu().numpy(), bits_of(sc), inp["perm"],
                              inp["signs"], inp["h"], 128)
    assert rel_fro(out_f64(out), y) < OUT_TOL
    out32 = rbp.int8_linear(xr, q, sc, 128, out_dtype=torch.float32)
    assert rel_fro(out_f64(out32), y) < 1e-3


@pytest.mark.parametrize("M,N", [(1, 7), (33, 129), (257, 300)])
def test_int8_linear_ragged(gpu_lib, M, N):
    rbp = gpu_lib
    inp, rot = _setup(rbp, M=M, N=N)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    bias = torch.from_numpy(np.random.default_rng(2).standard_normal(N).astype(np.float32)).cuda()
    out = rbp.int8_linear(xr, q, sc, 128, bias=bias, out_dtype=torch.float32)
    y, _ = oracle.int8_linear(as_f64(inp["X"]), q.cpu().numpy(), bits_of(sc), inp["perm"],
                              inp["signs"], inp["h"], 128)
    assert rel_fro(out_f64(out), y + bias.cpu().numpy()) < OUT_TOL


# Products with at least 128 tiles of 256 x 256 take the LDS-staged kernel;
# (4096, 2049, 384) has an odd number of scale entries and takes the
# register-fed kernel instead.  On the GPU's own fp16 x' the result differs
# from the exact product only by the fp16 rounding of each decoded weight
# (relative <= 2^-11) and fp32 accumulation.
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
def test_int8_linear_staged_tiles(gpu_lib, M, N, K):
    from oracle.int8 import int8_linear_rotated
    rbp = gpu_lib
    inp = synth.make(3, M=M, N=N, K=K, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    bias = torch.from_numpy(np.random.default_rng(3).standard_normal(N).astype(np.float32)).cuda()
    x16 = oracle.f16_bits_to_f64(bits_of(xr))
    y = int8_linear_rotated(x16, q.cpu().numpy(), bits_of(sc), 128) + bias.cpu().numpy()
    out32 = rbp.int8_linear(xr, q, sc, 128, bias=bias, out_dtype=torch.float32)
    assert rel_fro(out_f64(out32), y) < 2.0 ** -11
    out16 = rbp.int8_linear(xr, q, sc, 128, bias=bias)
    assert rel_fro(out_f64(out16), y) < OUT_TOL


@pytest.mark.parametrize("M,N,K", [(16, 1000, 2048), (9, 37, 4096), (3, 40000, 1024)])
def test_int8_narrow_bf16_bias_deterministic(gpu_lib, M, N, K):
    """The slab-walking kernel (up to 16 tokens) with a bf16 bias, into both
    output types, against the exact product on the GPU's own fp16 x' plus the
    bias's bf16 value; two launches give identical bits (the eight waves'
    partials are added in a fixed order)."""
    from oracle.int8 import int8_linear_rotated
    rbp = gpu_lib
    inp = synth.make(3, M=M, N=N, K=K, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    b32 = np.random.default_rng(4).standard_normal(N).astype(np.float32)
    bias = torch.from_numpy(b32).cuda().to(torch.bfloat16)
    bias_f64 = bias.float().cpu().numpy().astype(np.float64)
    y = int8_linear_rotated(oracle.f16_bits_to_f64(bits_of(xr)), q.cpu().numpy(), bits_of(sc), 128) + bias_f64
    out32 = rbp.int8_linear(xr, q, sc, 128, bias=bias, out_dtype=torch.float32)
    assert rel_fro(out_f64(out32), y) < 2.0 ** -11
    out16 = rbp.int8_linear(xr, q, sc, 128, bias=bias)
    assert rel_fro(out_f64(out16), y) < OUT_TOL
    again = rbp.int8_linear(xr, q, sc, 128, bias=bias)
    assert torch.equal(out16, again)


def test_int8_workload_full_size_sampled(gpu_lib):
    """The int8 workload at its full size (16384 tokens, 4096 -> 4096, h = 128)
    in the launch the benchmark times: sampled outputs against the literal
    dequantize -> inverse-rotate -> X W^T oracle, and against the exact
    product on the GPU's own fp16 x'."""
    from oracle.int8 import int8_linear_rotated
    rbp = gpu_lib
    inp, rot = _setup(rbp, M=16384, N=4096)
    q, sc = rbp.int8_pack_weights(rot, to_dev(inp["W"]), 128)
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    out = rbp.int8_linear(xr, q, sc, 128)
    g = np.random.default_rng(8)
    ms = np.sort(g.choice(16384, 64, replace=False))
    ns = np.sort(g.choice(4096, 96, replace=False))
    qn, scn = q[ns].cpu().numpy(), bits_of(sc[ns])
    got = out_f64(out[ms][:, ns])
    y, _ = oracle.int8_linear(as_f64(inp["X"][ms]), qn, scn, inp["perm"], inp["signs"],
                              inp["h"], 128)
    assert rel_fro(got, y) < OUT_TOL
    x16 = oracle.f16_bits_to_f64(bits_of(xr[ms]))
    y16 = int8_linear_rotated(x16, qn, scn, 128)
    assert rel_fro(got, y16) < OUT_TOL
