"""Edge cases of the hot path on the GPU: the longest rows the library takes,
empty batches at every entry point, and shapes the boundary must refuse.

The longest row is d = 16384 (64 blocks of 256, or 128 of 128): one
workgroup of four waves per row stages it once in LDS there (OrbitQuant
page, Method: the rotation and quantizer apply per token, whatever its
length).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import int4
from parity import as_f64, bits_of, check_bf16_norms, check_group_codes, check_indices, to_dev

pytestmark = pytest.mark.gpu

D_MAX = 16384


@pytest.mark.parametrize("h", [256, 128])
def test_quant_act_longest_rows(gpu_lib, h):
    rbp = gpu_lib
    perm, signs = synth.rotation_params(D_MAX, 7 + h)
    g = np.random.default_rng(h)
    X = synth.f32_to_bf16_bits(g.standard_normal((24, D_MAX)).astype(np.float32))
    X[5] = 0                                           # a zero token
    rot = rbp.Rotation(perm, signs, h)
    cb = rbp.Codebook(D_MAX, 4)
    ref_cb = oracle.codebook(4)
    idx, s, xr = rbp.quant_act(rot, cb, to_dev(X), synth.EPS, debug_xrot=True)
    torch.cuda.synchronize()
    ref = oracle.quant_act(as_f64(X), perm, signs, h, ref_cb, 4, synth.EPS)
    xr = xr.cpu().numpy().astype(np.float64)
    num = np.linalg.norm(xr - ref["xrot"], axis=1)
    den = np.maximum(np.linalg.norm(ref["xrot"], axis=1), 1e-300)
    assert np.all(num / den <= 1e-5)
    s = s.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s - ref["s"]) <= 1e-6 * ref["s"]) and s[5] == 0
    check_indices(idx, 4, D_MAX, ref["u"], ref_cb["thresholds"], f"d{D_MAX}-h{h}")
    # the plain rotation at the same length
    y = rbp.rotate(rot, to_dev(X), out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert np.all(np.linalg.norm(y - ref["xrot"], axis=1) <= 1e-5 * den)


@pytest.mark.parametrize("f32", [False, True])
def test_weight_packs_longest_rows(gpu_lib, f32):
    # fp32 rows of 16384: 128 KiB of x and -x in LDS plus the gather scratch
    rbp = gpu_lib
    perm, signs = synth.rotation_params(D_MAX, 3)
    g = np.random.default_rng(9)
    W = (0.02 * g.standard_normal((40, D_MAX))).astype(np.float32)
    if not f32:
        W = synth.f32_to_bf16_bits(W)
    rot = rbp.Rotation(perm, signs, 256)
    # codebook codes and norms
    cb = rbp.Codebook(D_MAX, 2)
    ref_cb = oracle.codebook(2)
    idx, r = rbp.pack_weights(rot, cb, to_dev(W))
    ref = oracle.pack_weights(as_f64(W), perm, signs, 256, ref_cb, 2)
    check_indices(idx, 2, D_MAX, ref["u"], ref_cb["thresholds"], "w2-longest")
    check_bf16_norms(bits_of(r), ref["r"], "w2-longest")
    # int8 and int4 group codes and fp16 scales
    for mode in ("int8", "int4"):
        if mode == "int8":
            q, sc = rbp.int8_pack_weights(rot, to_dev(W), 128)
            got, qmax = q.cpu().numpy(), 127
        else:
            q, sc = rbp.int4_pack_weights(rot, to_dev(W), 128)
            got, qmax = int4.unpack_nibbles(q.cpu().numpy(), D_MAX), 7
        check_group_codes(got, bits_of(sc), ref["wrot"], 128, qmax, f"{mode}-longest")


def test_empty_batches(gpu_lib):
    """Zero tokens (or zero weight rows) at every entry point: empty outputs,
    no error and nothing launched."""
    rbp = gpu_lib
    inp = synth.make(2, M=4, N=4)
    d = inp["X"].shape[1]
    rot = rbp.Rotation(inp["perm"], inp["signs"], inp["h"])
    cb = rbp.Codebook(d, 4)
    X0 = to_dev(inp["X"])[:0]
    idx, s = rbp.quant_act(rot, cb, X0)
    assert idx.shape == (0, d // 2) and s.shape == (0,)
    assert rbp.rotate(rot, X0).shape == (0, d)
    iw, r = rbp.pack_weights(rot, cb, X0)
    assert iw.shape == (0, d // 2) and r.shape == (0,)
    q8, s8 = rbp.int8_pack_weights(rot, X0, 128)
    q4, s4 = rbp.int4_pack_weights(rot, X0, 128)
    assert q8.shape == (0, d) and q4.shape == (0, d // 2) and s8.shape == (0, d // 128)
    # linear layers with an empty side
    W = to_dev(inp["W"])
    xr = rbp.rotate(rot, to_dev(inp["X"]), torch.float16)
    q8, s8 = rbp.int8_pack_weights(rot, W, 128)
    q4, s4 = rbp.int4_pack_weights(rot, W, 128)
    assert rbp.int8_linear(xr[:0], q8, s8, 128).shape == (0, 4)
    assert rbp.int8_linear(xr, q8[:0], s8[:0], 128).shape == (4, 0)
    assert rbp.int4_linear(xr[:0], q4, s4, 128).shape == (0, 4)
    assert rbp.int4_linear(xr, q4[:0], s4[:0], 128).shape == (4, 0)
    ia, sa = rbp.quant_act(rot, cb, to_dev(inp["X"]))
    iw, r = rbp.pack_weights(rot, cb, W)
    assert rbp.qlinear(ia, sa, cb, iw[:0], r[:0], cb, d).shape == (4, 0)
    torch.cuda.synchronize()


def test_rejects_rows_out_of_range(gpu_lib):
    """Shapes the boundary refuses on the host, before any launch."""
    rbp = gpu_lib
    # one block beyond the longest row
    d = D_MAX + 256
    perm, signs = synth.rotation_params(d, 1)
    rot = rbp.Rotation(perm, signs, 256)
    X = torch.zeros((2, d), dtype=torch.bfloat16, device="cuda")
    cb = rbp.Codebook(D_MAX, 4)
    with pytest.raises(rbp.OrbitError):
        rbp.quant_act(rot, cb, X)
    with pytest.raises(rbp.OrbitError):
        rbp.rotate(rot, X)
    # blocks longer than 1024 only for rows up to 4096
    perm, signs = synth.rotation_params(8192, 2)
    rot = rbp.Rotation(perm, signs, 2048)
    with pytest.raises(rbp.OrbitError):
        rbp.rotate(rot, torch.zeros((2, 8192), dtype=torch.bfloat16, device="cuda"))
    # d must be a multiple of h
    perm, signs = synth.rotation_params(3072, 3)
    rot = rbp.Rotation(perm, signs, 2048)
    with pytest.raises(rbp.OrbitError):
        rbp.rotate(rot, torch.zeros((2, 3072), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
