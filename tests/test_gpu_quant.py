"""GPU parity of the fused rotate + quantize kernels against the oracle.

Checks (OrbitQuant page, Method): x' = Pi x within 1e-5 relative per token,
s = ||x'|| within 1e-6, codebook indices bit-exact except where the rotated
coordinate lies within 1e-6 of a decision threshold (fraction < 1e-5), and
stored bf16 row norms bit-exact except within 1e-6 of a bf16 rounding tie.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import as_f64, bits_of, check_bf16_norms, check_indices, to_dev

pytestmark = pytest.mark.gpu

EPS = synth.EPS


def _run_act(rbp, X, perm, signs, h, bits, label, marginal="gauss"):
    d = X.shape[1]
    rot = rbp.Rotation(perm, signs, h)
    cb = rbp.Codebook(d, bits, marginal=marginal)
    ref_cb = oracle.codebook(bits) if marginal == "gauss" else oracle.codebook_sphere(bits, d)
    idx, s, xr = rbp.quant_act(rot, cb, to_dev(X), EPS, debug_xrot=True)
    torch.cuda.synchronize()
    ref = oracle.quant_act(as_f64(X), perm, signs, h, ref_cb, bits, EPS)
    xr = xr.cpu().numpy().astype(np.float64)
    num = np.linalg.norm(xr - ref["xrot"], axis=1)
    den = np.maximum(np.linalg.norm(ref["xrot"], axis=1), 1e-300)
    assert np.all(num / den <= 1e-5), f"{label}: x' error {np.max(num / den)}"
    s = s.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s - ref["s"]) <= 1e-6 * ref["s"]), f"{label}: s"
    stats, got = check_indices(idx, bits, d, ref["u"], ref_cb["thresholds"], label)
    return stats


CASES = [  # (label, workload, rows, bits)
    ("tiny-f32-h64-a4", 1, 64, 4),
    ("image-h128-a4", 2, 333, 4),
    ("mlp-up-h256-a4", 4, 200, 4),
    ("video-h128-a6", 5, 300, 6),
]


@pytest.mark.parametrize("label,cfg,rows,bits", CASES, ids=[c[0] for c in CASES])
def test_quant_act_workloads(gpu_lib, label, cfg, rows, bits):
    inp = synth.make(cfg, M=rows, N=8)
    _run_act(gpu_lib, inp["X"], inp["perm"], inp["signs"], inp["h"], bits, label)


@pytest.mark.parametrize("bits", [1, 2, 3, 8])
def test_quant_act_other_widths(gpu_lib, bits):
    inp = synth.make(2, M=96, N=8)
    _run_act(gpu_lib, inp["X"], inp["perm"], inp["signs"], inp["h"], bits, f"a{bits}")


@pytest.mark.parametrize("cfg,bits", [(1, 4), (2, 4), (2, 3), (5, 6)])
def test_quant_act_sphere_codebook(gpu_lib, cfg, bits):
    # the codebook of the exact sphere marginal f_d: the kernels read only
    # its float32 thresholds, so parity is the same as for N(0,1) tables
    inp = synth.make(cfg, M=128, N=8)
    _run_act(gpu_lib, inp["X"], inp["perm"], inp["signs"], inp["h"], bits,
             f"sphere-cfg{cfg}-a{bits}", marginal="sphere")


def test_quant_act_long_rows(gpu_lib):
    # d = 12288 (the MLP down projection input, 48 blocks of 256): rows longer
    # than 4096 take the two-pass path
    inp = synth.make(4, M=8)
    g = np.random.default_rng(5)
    X = synth.f32_to_bf16_bits(g.standard_normal((40, 12288)).astype(np.float32))
    _run_act(gpu_lib, X, inp["perm2"], inp["signs2"], 256, 4, "down-d12288")


# (512, 64), (1536, 128), (2560, 256), (6144, 128): bf16 rows with h = 64,
# 128, 256 whose width the matrix-core kernels do not take, so the
# transposed-gather butterfly kernels (one wave per row, or one workgroup
# per row past 4096) run them
@pytest.mark.parametrize("d,h", [(1040, 16), (48, 16), (3072, 32), (3072, 1024), (1024, 1024),
                                 (2048, 2048), (4096, 4096), (4096, 2048),
                                 (512, 64), (1536, 128), (2560, 256), (6144, 128)])
def test_quant_act_shapes(gpu_lib, d, h):
    perm, signs = synth.rotation_params(d, 100 + d + h)
    g = np.random.default_rng(d + h)
    X = synth.f32_to_bf16_bits(g.standard_normal((70, d)).astype(np.float32))
    _run_act(gpu_lib, X, perm, signs, h, 4, f"d{d}-h{h}")


# bf16 rows with h = 64, 128, 256 and d = 1024 .. 4096 take the matrix-core
# kernels (H_32 as bf16 MFMAs, the group stages in registers and, for
# h = 256, between lanes l and l ^ 16); 77 rows leave waves without a row
@pytest.mark.parametrize("d,h,bits", [(1024, 64, 4), (2048, 256, 2), (4096, 256, 6), (4096, 64, 8),
                                      (3072, 256, 3), (2048, 128, 8), (1024, 256, 4)])
def test_quant_act_matrix_core_shapes(gpu_lib, d, h, bits):
    perm, signs = synth.rotation_params(d, 7 * d + h)
    g = np.random.default_rng(d + 3 * h + bits)
    X = synth.f32_to_bf16_bits(g.standard_normal((77, d)).astype(np.float32))
    X[11] = 0
    _run_act(gpu_lib, X, perm, signs, h, bits, f"mfma-d{d}-h{h}-a{bits}")


@pytest.mark.parametrize("d,h", [(2048, 128), (12288, 256), (1024, 64)])
def test_quant_act_identity_permutation(gpu_lib, d, h):
    # pi = identity (Block-RHT, or the MLP down layer with pi folded into the
    # up layer): the plan builder flags it and the matrix-core kernels read each
    # fragment as contiguous bytes instead of gathering it
    _, signs = synth.rotation_params(d, 17 + d)
    perm = np.arange(d, dtype=np.int32)
    g = np.random.default_rng(h + d)
    X = synth.f32_to_bf16_bits(g.standard_normal((70, d)).astype(np.float32))
    rot = gpu_lib.Rotation(perm, signs, h)
    assert rot.struct.flags == gpu_lib.RPBH_IDENTITY
    _run_act(gpu_lib, X, perm, signs, h, 4, f"ident-d{d}-h{h}")


def test_quant_act_matrix_core_3072_wide(gpu_lib):
    # 3072-wide rows take the matrix-core kernel above 16 rows per compute
    # unit (4096 on MI355X): 4100 rows, a ragged last round of waves
    g = np.random.default_rng(41)
    perm, signs = synth.rotation_params(3072, 41)
    X = synth.f32_to_bf16_bits(g.standard_normal((4100, 3072)).astype(np.float32))
    _run_act(gpu_lib, X, perm, signs, 128, 4, "mfma-d3072-4100rows")


@pytest.mark.parametrize("d,h", [(1024, 64), (4096, 256)])
def test_weight_pack_matrix_core_shapes(gpu_lib, d, h):
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, 5 * d + h)
    g = np.random.default_rng(d + h)
    W = synth.f32_to_bf16_bits((0.03 * g.standard_normal((90, d))).astype(np.float32))
    rot = rbp.Rotation(perm, signs, h)
    cb = rbp.Codebook(d, 2)
    ref_cb = oracle.codebook(2)
    idx, r = rbp.pack_weights(rot, cb, to_dev(W))
    ref = oracle.pack_weights(as_f64(W), perm, signs, h, ref_cb, 2)
    check_indices(idx, 2, d, ref["u"], ref_cb["thresholds"], f"mfma-w-d{d}-h{h}")
    check_bf16_norms(bits_of(r), ref["r"], f"mfma-w-d{d}-h{h}")


@pytest.mark.parametrize("d", [2048, 4096])
def test_full_rht_rotate_and_weights(gpu_lib, d):
    """Full RHT (OrbitQuant page, Experiments: the rotation ablation), h = d:
    rotations and weight codes against the oracle's full_rht_rotate."""
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, 40 + d)
    g = np.random.default_rng(d)
    X = synth.f32_to_bf16_bits(g.standard_normal((48, d)).astype(np.float32))
    rot = rbp.Rotation(perm, signs, d)
    ref = oracle.full_rht_rotate(as_f64(X), perm, signs)
    for dt, tol in ((torch.float32, 1e-5), (torch.float16, 2e-3)):
        y = rbp.rotate(rot, to_dev(X), out_dtype=dt).cpu().numpy().astype(np.float64)
        err = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert np.all(err <= tol), f"full RHT d={d} {dt}: {err.max()}"
    cb = rbp.Codebook(d, 4)
    ref_cb = oracle.codebook(4)
    idx, r = rbp.pack_weights(rot, cb, to_dev(X))
    wref = oracle.pack_weights(as_f64(X), perm, signs, d, ref_cb, 4)
    check_indices(idx, 4, d, wref["u"], ref_cb["thresholds"], f"full-rht-w{d}")
    check_bf16_norms(bits_of(r), wref["r"], f"full-rht-w{d}")


def test_block_rht_identity_permutation(gpu_lib):
    # Block-RHT (the ablation's variant without the permutation)
    d = 3072
    _, signs = synth.rotation_params(d, 9)
    inp = synth.make(2, M=64, N=8)
    _run_act(gpu_lib, inp["X"], np.arange(d, dtype=np.int32), signs, 128, 4, "block-rht")


def test_zero_and_nan_tokens(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=8, N=8)
    X = inp["X"].copy()
    X[2] = 0                      # an all-zero token
    X[5, 17] = 0x7FC0             # a NaN coordinate
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    cb = rbp.Codebook(3072, 4)
    idx, s = rbp.quant_act(rot, cb, to_dev(X), EPS)
    s = s.cpu().numpy()
    assert s[2] == 0.0 and np.isnan(s[5]) and np.all(np.isfinite(np.delete(s, 5)))
    zero_codes = oracle.unpack_indices(idx[2:3].cpu().numpy(), 4, 3072)
    assert np.all(zero_codes == 7)            # u = 0 -> #{t_j < 0} = 7


def test_weight_pack_workloads(gpu_lib):
    rbp = gpu_lib
    for label, cfg, rows, bits, key in [("tiny-f32", 1, 256, 4, "W"), ("image", 2, 200, 4, "W"),
                                        ("mlp-up-w2", 4, 150, 2, "W"), ("video", 5, 130, 4, "W")]:
        inp = synth.make(cfg, M=8, N=rows)
        W = inp[key].copy()
        W[3] = 0                                     # a zero row: r = 0, u = 0
        d = W.shape[1]
        rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
        cb = rbp.Codebook(d, bits)
        ref_cb = oracle.codebook(bits)
        idx, r = rbp.pack_weights(rot, cb, to_dev(W))
        torch.cuda.synchronize()
        ref = oracle.pack_weights(as_f64(W), inp["perm"], inp["signs"], inp["h"], ref_cb, bits)
        check_indices(idx, bits, d, ref["u"], ref_cb["thresholds"], label)
        got_r = bits_of(r)
        check_bf16_norms(got_r, ref["r"], label)
        assert got_r[3] == 0


@pytest.mark.parametrize("d,h", [(1536, 128), (512, 64)])
def test_weight_pack_butterfly_widths(gpu_lib, d, h):
    # bf16 weight rows whose width the matrix-core kernels do not take
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, 11 * d + h)
    g = np.random.default_rng(5 * d + h)
    W = synth.f32_to_bf16_bits(g.standard_normal((90, d)).astype(np.float32))
    rot = rbp.Rotation(perm, signs, h)
    cb = rbp.Codebook(d, 4)
    ref_cb = oracle.codebook(4)
    idx, r = rbp.pack_weights(rot, cb, to_dev(W))
    torch.cuda.synchronize()
    ref = oracle.pack_weights(as_f64(W), perm, signs, h, ref_cb, 4)
    check_indices(idx, 4, d, ref["u"], ref_cb["thresholds"], f"w-d{d}-h{h}")
    check_bf16_norms(bits_of(r), ref["r"], f"w-d{d}-h{h}")


def test_weight_pack_long_rows(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(4, M=8)
    W = inp["W2"][:48]                           # down projection rows, d = 12288
    rot = rbp.Rotation(inp["perm2"], inp["signs2"], 256)
    cb = rbp.Codebook(12288, 2)
    idx, r = rbp.pack_weights(rot, cb, to_dev(W))
    ref_cb = oracle.codebook(2)
    ref = oracle.pack_weights(as_f64(W), inp["perm2"], inp["signs2"], 256, ref_cb, 2)
    check_indices(idx, 2, 12288, ref["u"], ref_cb["thresholds"], "down-w2")
    check_bf16_norms(bits_of(r), ref["r"], "down-w2")


def test_deterministic(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=256, N=8)
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    cb = rbp.Codebook(3072, 4)
    X = to_dev(inp["X"])
    a = rbp.quant_act(rot, cb, X, EPS)
    b = rbp.quant_act(rot, cb, X, EPS)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# Row counts past one row per wave (or per workgroup) of a full launch, so
# each wave (workgroup) loops over several rows with the next row's loads in
# flight: the rows and their codes are checked on a sample that includes the
# last rows of the batch and rows of every loop trip.
def _loop_rows(M, k=64, seed=0):
    g = np.random.default_rng(seed)
    rows = set(g.choice(M, k, replace=False).tolist()) | {0, 1, M - 2, M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("M,d,h,bits,ident", [
    (4096, 12288, 256, 4, True),     # the MLP down quantizer (pi folded away)
    (4096, 12288, 256, 4, False),
    (2300, 16384, 128, 4, False),
    (9000, 1024, 64, 4, False),      # one wave per row, several rows per wave
    (9000, 2048, 128, 6, False),
    (6200, 4096, 256, 2, False),
])
def test_quant_act_multi_row_loop(gpu_lib, M, d, h, bits, ident):
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, 3 * d + h + bits)
    if ident:
        perm = np.arange(d, dtype=np.int32)
    g = np.random.default_rng(d + M)
    X = synth.f32_to_bf16_bits(g.standard_normal((M, d)).astype(np.float32))
    rows = _loop_rows(M, seed=d)
    X[rows[3]] = 0                                        # a zero token in the sample
    rot = rbp.Rotation(perm, signs, h)
    cb = rbp.Codebook(d, bits)
    ref_cb = oracle.codebook(bits)
    idx, s = rbp.quant_act(rot, cb, to_dev(X), EPS)
    torch.cuda.synchronize()
    # every row's s against ||x|| (Pi is orthogonal: ||Pi x|| = ||x||)
    s = s.cpu().numpy().astype(np.float64)
    s_ref = np.linalg.norm(as_f64(X), axis=1)
    assert np.all(np.abs(s - s_ref) <= 1e-6 * s_ref)
    ref = oracle.quant_act(as_f64(X[rows]), perm, signs, h, ref_cb, bits, EPS)
    check_indices(idx[rows], bits, d, ref["u"], ref_cb["thresholds"], f"loop-{M}x{d}-h{h}")


@pytest.mark.parametrize("ident", [False, True])
def test_weight_pack_down_projection_full(gpu_lib, ident):
    """W_down of the MLP pair at its full size (3072 x 12288, 2-bit codes,
    h = 256): several rows per workgroup; every row's bf16 norm against the
    fp64 norm (||W Pi^T|| = ||W|| row by row), codes on sampled rows."""
    rbp = gpu_lib
    inp = synth.make(4, M=8)
    W = inp["W2"]
    N, d = W.shape
    perm = np.arange(d, dtype=np.int32) if ident else inp["perm2"]
    rot = rbp.Rotation(perm, inp["signs2"], 256)
    cb = rbp.Codebook(d, 2)
    idx, r = rbp.pack_weights(rot, cb, to_dev(W))
    torch.cuda.synchronize()
    check_bf16_norms(bits_of(r), np.linalg.norm(as_f64(W), axis=1), "w-down-full")
    rows = _loop_rows(N, seed=5)
    ref_cb = oracle.codebook(2)
    ref = oracle.pack_weights(as_f64(W[rows]), perm, inp["signs2"], 256, ref_cb, 2)
    check_indices(idx[rows], 2, d, ref["u"], ref_cb["thresholds"], "w-down-full")
    check_bf16_norms(bits_of(r)[rows], ref["r"], "w-down-full")
