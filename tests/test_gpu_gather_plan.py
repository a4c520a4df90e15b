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


def _row_byte(p, d):
    """Byte offset of coordinate p in the LDS row of the h = 128 / 256
    matrix-core kernels: two bytes per bf16 and, for rows of up to 12288
    coordinates, a 16-byte pad after every 64."""
    return 2 * p + (16 * (p // 64) if d <= 12288 else 0)


def _words_reference(perm, signs, h):
    """The documented matrix-core section (empty unless h is 64 .. 4096 and
    d % 512 == 0).  h = 64: word 4 (64 c + l) + q covers permuted
    coordinates k, k + 1 with k = 512 c + 32 (l % 16) + 8 (l // 16) + 2 q, at
    byte offsets 2 pi(k).  h = 128 / 256: word 4 (64 o + l) + q covers slots
    j = 2 q, 2 q + 1 of A operand o for lane l = 16 kq + r16, the permuted
    coordinate of slot j being 512 o + 128 (r16 // 4) + 32 kq + 4 j + r16 % 4
    (h = 128, and 512 .. 4096) or 1024 (o // 2) + 256 (r16 // 4) + 64 kq +
    8 j + 4 (o % 2) + r16 % 4 (h = 256), at the padded row's byte offsets."""
    d = perm.shape[0]
    if h not in (64, 128, 256, 512, 1024, 2048, 4096) or d % 512:
        return np.zeros(0, dtype=np.int64)
    out = np.zeros(d // 2, dtype=np.int64)

    def word(k0, k1, off):
        return (off(k0) | (int(signs[k0] < 0) << 15) | (off(k1) << 16) | (int(signs[k1] < 0) << 31))

    for o in range(d // 512):
        for lane in range(64):
            kq, r16 = divmod(lane, 16)
            for q in range(4):
                if h == 64:
                    k = 512 * o + 32 * r16 + 8 * kq + 2 * q
                    w = word(k, k + 1, lambda k: 2 * int(perm[k]))
                else:
                    ks = []
                    for j in (2 * q, 2 * q + 1):
                        if h != 256:
                            ks.append(512 * o + 128 * (r16 // 4) + 32 * kq + 4 * j + r16 % 4)
                        else:
                            ks.append(1024 * (o // 2) + 256 * (r16 // 4) + 64 * kq + 8 * j
                                      + 4 * (o % 2) + r16 % 4)
                    w = word(ks[0], ks[1], lambda k: _row_byte(int(perm[k]), d))
                out[4 * (64 * o + lane) + q] = w
    return out


def _scatter_reference(perm, signs, h):
    """The documented scatter section (h = 128 / 256 on rows of 1024, 2048,
    3072, 4096, 8192, 12288 or 16384 coordinates, else empty): entry i is
    the LDS byte offset 16 (64 o + l) + 2 j of the operand slot (o, l, j)
    whose permuted coordinate k (the slot order of the offset words) has
    pi(k) = i, with D_k in bit 15."""
    d = perm.shape[0]
    if h not in (128, 256) or d not in (1024, 2048, 3072, 4096, 8192, 12288, 16384):
        return np.zeros(0, dtype=np.int64)
    out = np.full(d, -1, dtype=np.int64)
    for o in range(d // 512):
        for lane in range(64):
            kq, r16 = divmod(lane, 16)
            for j in range(8):
                if h == 128:
                    k = 512 * o + 128 * (r16 // 4) + 32 * kq + 4 * j + r16 % 4
                else:
                    k = 1024 * (o // 2) + 256 * (r16 // 4) + 64 * kq + 8 * j + 4 * (o % 2) + r16 % 4
                out[int(perm[k])] = 16 * (64 * o + lane) + 2 * j + (int(signs[k] < 0) << 15)
    assert (out >= 0).all()
    return out


def _check_plan(rot, perm, signs, h, rounds):
    got = rot.gather.cpu().numpy()
    n = 1024 * rounds
    words = _words_reference(perm, signs, h)
    scat = _scatter_reference(perm, signs, h)
    nw = 2 * words.shape[0]
    assert got.shape == (n + nw + scat.shape[0],)
    assert np.array_equal(got[:n].view(np.uint16).astype(np.int64), _plan_reference(perm, signs, h, rounds))
    assert np.array_equal(got[n:n + nw].view(np.uint32).astype(np.int64), words)
    assert np.array_equal(got[n + nw:].view(np.uint16).astype(np.int64), scat)


@pytest.mark.parametrize("d,h", [(3072, 128), (1024, 64), (2048, 256), (3072, 256), (512, 32), (96, 16),
                                 (4096, 4096), (2048, 512)])
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
    (2, 3072, 128, 4, False),   # packed-code matrix-core kernel: words from the plan or from pi
    (2, 1024, 64, 2, False),    # first matrix-core kernel (h = 64)
    (2, 2048, 256, 6, False),
    (2, 4096, 128, 3, False),   # 3-bit codes with h = 128: first matrix-core kernel, words from pi
    (2, 12288, 256, 4, False),  # packed-code kernel, four waves per row
    (2, 8192, 256, 3, False),
    (2, 4096, 4096, 4, False),  # full RHT: h = 128 factor on the matrix cores, block bits after
    (2, 2048, 1024, 6, False),
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


def test_plan_refuses_a_perm_that_is_not_a_permutation(gpu_lib):
    """The scatter section has one entry per input coordinate, so the plan
    builder checks that perm is a permutation before it launches anything."""
    perm, signs = synth.rotation_params(1024, 5)
    bad = perm.copy()
    bad[3] = bad[7]                       # one index twice, one missing
    with pytest.raises(gpu_lib.OrbitError, match="status 1"):
        gpu_lib.Rotation(bad, signs, 128)
    out_of_range = perm.copy()
    out_of_range[0] = 1024
    with pytest.raises(gpu_lib.OrbitError, match="status 1"):
        gpu_lib.Rotation(out_of_range, signs, 128)


@pytest.mark.parametrize("d,h,bits", [(3072, 128, 4), (2048, 128, 6), (1024, 256, 2), (3072, 256, 4),
                                      (4096, 128, 8), (8192, 256, 4), (16384, 128, 4)])
def test_scatter_and_gather_forms_agree(gpu_lib, d, h, bits):
    """The activation quantizer's two forms on a permuting rotation: with the
    plan the lanes scatter the row into operand order, without it they
    gather their operands; the codes, norms and x' must be bit-identical
    (the same MFMA operands in the same order), on enough rows that waves
    loop over several."""
    rbp = gpu_lib
    perm, signs = synth.rotation_params(d, d + h + bits)
    g = np.random.default_rng(d + bits)
    M = 2100 if d <= 4096 else 700
    X = to_dev(synth.f32_to_bf16_bits(g.standard_normal((M, d)).astype(np.float32)))
    cb = rbp.Codebook(d, bits)
    with_plan = rbp.Rotation(perm, signs, h)
    without = rbp.Rotation(perm, signs, h, plan=False)
    i1, s1 = rbp.quant_act(with_plan, cb, X, synth.EPS)
    i2, s2 = rbp.quant_act(without, cb, X, synth.EPS)
    i3, s3, x3 = rbp.quant_act(with_plan, cb, X[:300], synth.EPS, debug_xrot=True)
    i4, s4, x4 = rbp.quant_act(without, cb, X[:300], synth.EPS, debug_xrot=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(i3, i4) and torch.equal(x3.view(torch.int32), x4.view(torch.int32))
    assert torch.equal(i3, i1[:300])
