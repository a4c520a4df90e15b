"""The rotation's gather plan (orbit_rpbh_build_gather): its layout, and that
every row kernel gives bit-identical results with and without it.

The plan is derived data of the rotation (OrbitQuant page, Method: y_k =
D_k x[pi(k)] for the permuted, sign-flipped coordinates); results must not
depend on whether a kernel reads it or derives its offsets from pi and the
signs itself.
"""
import numpy as np
import pytest
import torch

import synth
from parity import to_dev

pytestmark = pytest.mark.gpu


def _plan_reference(perm, signs, h, rounds=4):
    """The documented layout: entry r*1024 + l*16 + e."""
    d = perm.shape[0]
    out = np.zeros(1024 * rounds, dtype=np.int64)
    T = h // 16 if h in (64, 128, 256) else None
    for r in range(rounds):
        for lane in range(64):
            s = 64 * r + lane
            if s >= d // 16:
                continue
            for e in range(16):
                if T is None:
                    k = 16 * s + e
                else:
                    G = 16 // T
                    p = s % T
                    t, i = divmod(e, G)
                    k = 16 * (s - p) + 16 * t + G * p + i
                out[r * 1024 + lane * 16 + e] = perm[k] + (d if signs[k] < 0 else 0)
    return out


def _words_reference(perm, signs, h):
    """The documented matrix-core section: word 4 (64 c + l) + q covers
    permuted coordinates k, k + 1 with k = 512 c + 32 (l % 16) + 8 (l // 16)
    + 2 q; empty unless h is 64, 128 or 256 and d % 512 == 0."""
    d = perm.shape[0]
    if h not in (64, 128, 256) or d % 512:
        return np.zeros(0, dtype=np.int64)
    out = np.zeros(d // 2, dtype=np.int64)
    for c in range(d // 512):
        for lane in range(64):
            for q in range(4):
                k = 512 * c + 32 * (lane % 16) + 8 * (lane // 16) + 2 * q
                out[4 * (64 * c + lane) + q] = (2 * int(perm[k]) | (int(signs[k] < 0) << 15)
                                                | (2 * int(perm[k + 1])) << 16
                                                | (int(signs[k + 1] < 0) << 31))
    return out


def _check_plan(rot, perm, signs, h, rounds):
    got = rot.gather.cpu().numpy()
    n = 1024 * rounds
    words = _words_reference(perm, signs, h)
    assert got.shape == (n + 2 * words.shape[0],)
    assert np.array_equal(got[:n].view(np.uint16).astype(np.int64), _plan_reference(perm, signs, h, rounds))
    assert np.array_equal(got[n:].view(np.uint32).astype(np.int64), words)


@pytest.mark.parametrize("d,h", [(3072, 128), (1024, 64), (2048, 256), (512, 32), (96, 16)])
def test_plan_layout(gpu_lib, d, h):
    perm, signs = synth.rotation_params(d, 7 + d + h)
    rot = gpu_lib.Rotation(perm, signs, h)
    torch.cuda.synchronize()
    _check_plan(rot, perm, signs, h, 4)


def test_plan_for_long_rows(gpu_lib):
    d, h = 12288, 256
    perm, signs = synth.rotation_params(d, 3)
    rot = gpu_lib.Rotation(perm, signs, h)
    torch.cuda.synchronize()
    _check_plan(rot, perm, signs, h, 12)


@pytest.mark.parametrize("cfg,K,h,bits,f32", [
    (2, 3072, 128, 4, False),   # transposed-gather kernel, bf16
    (2, 1024, 64, 2, False),    # matrix-core kernel: words from the plan or from pi
    (2, 2048, 256, 6, False),
    (2, 4096, 128, 3, False),
    (2, 12288, 256, 4, False),  # matrix-core long-row kernel
    (2, 512, 32, 4, False),     # consecutive order, bf16
    (2, 3072, 128, 1, False),   # 1-bit codes: consecutive kernel, plan order differs -> unused
    (1, 256, 64, 4, True),      # fp32 rows: consecutive kernel, plan order differs -> unused
    (1, 256, 32, 3, True),      # fp32 rows, consecutive plan used
])
def test_quant_act_same_with_and_without_plan(gpu_lib, cfg, K, h, bits, f32):
    rbp = gpu_lib
    inp = synth.make(cfg, M=300, N=8, K=K, h=h)
    X = to_dev(inp["X"])
    if f32 and X.dtype != torch.float32:
        X = X.float()
    cb = rbp.Codebook(K, bits)
    with_plan = rbp.Rotation(inp["perm"], inp["signs"], h)
    without = rbp.Rotation(inp["perm"], inp["signs"], h, plan=False)
    assert with_plan.gather is not None and without.gather is None
    i1, s1, x1 = rbp.quant_act(with_plan, cb, X, synth.EPS, debug_xrot=True)
    i2, s2, x2 = rbp.quant_act(without, cb, X, synth.EPS, debug_xrot=True)
    # the production instances (no debug copy of x') as well
    i3, s3 = rbp.quant_act(with_plan, cb, X, synth.EPS)
    i4, s4 = rbp.quant_act(without, cb, X, synth.EPS)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(i3, i4) and torch.equal(i1, i3)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(s3.view(torch.int32), s4.view(torch.int32))
    assert torch.equal(x1.view(torch.int32), x2.view(torch.int32))


@pytest.mark.parametrize("h", [128, 32])
def test_weight_rotate_int8_same_with_and_without_plan(gpu_lib, h):
    rbp = gpu_lib
    inp = synth.make(2, M=64, N=200, K=1024, h=h)
    W = to_dev(inp["W"])
    X = to_dev(inp["X"])
    a = rbp.Rotation(inp["perm"], inp["signs"], h)
    b = rbp.Rotation(inp["perm"], inp["signs"], h, plan=False)
    cw = rbp.Codebook(1024, 4)
    ia, ra = rbp.pack_weights(a, cw, W)
    ib, rb = rbp.pack_weights(b, cw, W)
    assert torch.equal(ia, ib) and torch.equal(ra.view(torch.int16), rb.view(torch.int16))
    for dt in (torch.float32, torch.float16):
        ya = rbp.rotate(a, X, out_dtype=dt)
        yb = rbp.rotate(b, X, out_dtype=dt)
        assert torch.equal(ya, yb)
    qa, sa = rbp.int8_pack_weights(a, W)
    qb, sb = rbp.int8_pack_weights(b, W)
    assert torch.equal(qa, qb) and torch.equal(sa.view(torch.int16), sb.view(torch.int16))
