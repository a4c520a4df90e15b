"""GPU parity of the codebook-decode GEMM against the oracle on the same codes.

OrbitQuant page, Method: out[m, n] = r_n s_m <Q(w~_n), Q(x~_m)>.  The oracle
takes the GPU's own codes (indices, s, bf16 r) and its own fp64 codebook and
computes the product in fp64; the layer output must agree within 2e-3
relative Frobenius.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import OUT_TOL, as_f64, bits_of, out_f64, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _codes(rbp, X, W, perm, signs, h, ba, bw):
    d = X.shape[1]
    rot = rbp.Rotation(perm, signs, h)
    ca, cw = rbp.Codebook(d, ba), rbp.Codebook(d, bw)
    ia, s = rbp.quant_act(rot, ca, to_dev(X), synth.EPS)
    iw, r = rbp.pack_weights(rot, cw, to_dev(W))
    return rot, ca, cw, ia, s, iw, r


def _oracle_out(ia, s, iw, r, ba, bw, K, bias=None):
    A = oracle.unpack_indices(ia.cpu().numpy(), ba, K)
    B = oracle.unpack_indices(iw.cpu().numpy(), bw, K)
    return oracle.qlinear_codes(A, s.cpu().numpy(), oracle.codebook(ba)["centroids"], B,
                                bits_of(r), oracle.codebook(bw)["centroids"], K, bias)


CASES = [  # label, workload, M, N, act bits, weight bits, out dtype
    ("tiny-w4a4-f32", 1, 64, 256, 4, 4, torch.float32),
    ("image-w4a4", 2, 300, 200, 4, 4, torch.bfloat16),
    ("mlp-up-w2a4", 4, 260, 300, 4, 2, torch.bfloat16),
    ("video-w4a6", 5, 300, 130, 6, 4, torch.bfloat16),
]


@pytest.mark.parametrize("label,cfg,M,N,ba,bw,odt", CASES, ids=[c[0] for c in CASES])
def test_qlinear_workloads(gpu_lib, label, cfg, M, N, ba, bw, odt):
    rbp = gpu_lib
    inp = synth.make(cfg, M=M, N=N)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"],
                                     inp["h"], ba, bw)
    K = inp["K"]
    out = rbp.qlinear(ia, s, ca, iw, r, cw, K, out_dtype=odt)
    ref = _oracle_out(ia, s, iw, r, ba, bw, K)
    err = rel_fro(out_f64(out), ref)
    assert err < OUT_TOL, f"{label}: {err}"
    if odt == torch.float32:
        assert err < 5e-4  # no output rounding: only the fp16 codebook values remain


@pytest.mark.parametrize("ba,bw", [(2, 2), (3, 3), (8, 8), (8, 4), (4, 8), (6, 6), (3, 4), (2, 6)])
def test_qlinear_widths(gpu_lib, ba, bw):
    rbp = gpu_lib
    inp = synth.make(2, M=70, N=90, K=256, h=64)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"], 64, ba, bw)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, 256, out_dtype=torch.float32)
    ref = _oracle_out(ia, s, iw, r, ba, bw, 256)
    assert rel_fro(out_f64(out), ref) < OUT_TOL


# K over the kernel's k-chunks (128 for 2- and 4-bit pairs, 64 otherwise):
# an odd count of 128-chunks runs its first chunk ahead of the paired loop.
@pytest.mark.parametrize("ba,bw,K", [(4, 4, 128), (4, 4, 384), (2, 4, 640), (4, 2, 1152),
                                     (6, 4, 384), (3, 3, 640), (8, 4, 384)])
def test_qlinear_chunk_counts(gpu_lib, ba, bw, K):
    rbp = gpu_lib
    inp = synth.make(2, M=300, N=260, K=K, h=128)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"], 128, ba, bw)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, K, out_dtype=torch.float32)
    ref = _oracle_out(ia, s, iw, r, ba, bw, K)
    assert rel_fro(out_f64(out), ref) < OUT_TOL, (ba, bw, K)


@pytest.mark.parametrize("M,N", [(1, 1), (1, 300), (17, 5), (257, 193), (513, 385)])
def test_qlinear_ragged(gpu_lib, M, N):
    rbp = gpu_lib
    inp = synth.make(2, M=M, N=N, K=512, h=128)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"], 128, 4, 4)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, 512, out_dtype=torch.float32)
    ref = _oracle_out(ia, s, iw, r, 4, 4, 512)
    assert rel_fro(out_f64(out), ref) < OUT_TOL


def test_qlinear_bias(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=64, N=96, K=512, h=128)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"], 128, 4, 4)
    b = np.random.default_rng(1).standard_normal(96).astype(np.float32)
    for bias in (torch.from_numpy(b).cuda(), torch.from_numpy(b).cuda().to(torch.bfloat16)):
        out = rbp.qlinear(ia, s, ca, iw, r, cw, 512, bias=bias, out_dtype=torch.float32)
        ref = _oracle_out(ia, s, iw, r, 4, 4, 512, bias.float().cpu().numpy())
        assert rel_fro(out_f64(out), ref) < OUT_TOL


def test_zero_token_zero_row_and_nan(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=16, N=32, K=512, h=128)
    X, W = inp["X"].copy(), inp["W"].copy()
    X[3] = 0
    X[7, 5] = 0x7FC0
    W[4] = 0
    _, ca, cw, ia, s, iw, r = _codes(rbp, X, W, inp["perm"], inp["signs"], 128, 4, 4)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, 512, out_dtype=torch.float32).cpu().numpy()
    assert np.all(out[3] == 0)                       # zero token: s = 0
    assert np.all(np.delete(out[:, 4], 7) == 0)      # zero weight row: r = 0
    assert np.all(np.isnan(out[7]))                  # NaN token: NaN row (0 * NaN too)
    rest = np.delete(np.delete(out, [3, 7], axis=0), 4, axis=1)
    assert np.all(np.isfinite(rest))


def test_empty(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=4, N=4, K=256, h=64)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"], 64, 4, 4)
    out = rbp.qlinear(ia[:0], s[:0], ca, iw, r, cw, 256)
    assert out.shape == (0, 4)


# (label, workload, act bits, weight bits): full-size layers in the launch
# configurations the benchmark times.  The video layer and the wide-activation
# pairs take the 2 x 4 wave tile (the costlier token decode on the short
# side); the image and MLP layers the 4 x 3 tile.
FULL = [("image-w4a4", 2, 4, 4), ("video-w4a6", 5, 6, 4), ("mlp-up-w2a4", 4, 4, 2),
        ("image-w2a3", 2, 3, 2), ("image-w4a8", 2, 8, 4)]


@pytest.mark.parametrize("label,cfg,ba,bw", FULL, ids=[c[0] for c in FULL])
def test_layer_full_size_sampled(gpu_lib, label, cfg, ba, bw):
    """A layer at its full size; the oracle recomputes sampled outputs and
    sampled tokens' codes one by one."""
    rbp = gpu_lib
    inp = synth.make(cfg)
    K = inp["K"]
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"],
                                     inp["h"], ba, bw)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, K)
    g = np.random.default_rng(0)
    ms = np.sort(g.choice(inp["M"], 48, replace=False))
    ns = np.sort(g.choice(inp["N"], 64, replace=False))
    sub = _oracle_out(ia[ms], s[ms], iw[ns], r[ns], ba, bw, K)
    got = out_f64(out[ms][:, ns])
    assert rel_fro(got, sub) < OUT_TOL, label
    # the sampled tokens' codes against the oracle's rotation + quantizer
    from parity import check_indices
    ref = oracle.quant_act(as_f64(inp["X"][ms]), inp["perm"], inp["signs"], inp["h"],
                           oracle.codebook(ba), ba, synth.EPS)
    check_indices(ia[ms], ba, K, ref["u"], oracle.codebook(ba)["thresholds"], label)


@pytest.mark.parametrize("cfg,ba,bw,M,N,TN", [(5, 6, 4, 4608, 8192 + 96, 384),
                                               (5, 6, 4, 6144, 8192 + 96, 256),
                                               (5, 6, 4, 4096, 12032, 512),
                                               (4, 4, 2, 12800, 4096 + 40, 512)])
def test_wide_tile_ragged(gpu_lib, cfg, ba, bw, M, N, TN):
    """Products with enough tiles to take the wide wave tiles, for 6-bit
    tokens and 4-bit weights: 2 x 6 (128 x 384 per workgroup), 4 x 4 (256 x
    256) and 2 x 8 (128 x 512, where a ragged last column gives 752 tiles of
    256 x 256 and 768 of 128 x 512); 2 x 8 for 2-bit weights; each with a
    ragged last column of tiles.  Sampled tokens against every output
    column of the last two tile columns and sampled ones elsewhere."""
    rbp = gpu_lib
    inp = synth.make(cfg, M=M, N=N)
    K = inp["K"]
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"],
                                     inp["h"], ba, bw)
    out = rbp.qlinear(ia, s, ca, iw, r, cw, K)
    g = np.random.default_rng(5)
    ms = np.sort(g.choice(M, 40, replace=False))
    tail = np.arange((N // TN - 1) * TN, N)
    ns = np.unique(np.concatenate([tail, g.choice(N, 64, replace=False)]))
    sub = _oracle_out(ia[ms], s[ms], iw[ns], r[ns], ba, bw, K)
    assert rel_fro(out_f64(out[ms][:, ns]), sub) < OUT_TOL


def test_deterministic(gpu_lib):
    rbp = gpu_lib
    inp = synth.make(2, M=300, N=200)
    _, ca, cw, ia, s, iw, r = _codes(rbp, inp["X"], inp["W"], inp["perm"], inp["signs"],
                                     inp["h"], 4, 4)
    a = rbp.qlinear(ia, s, ca, iw, r, cw, inp["K"])
    b = rbp.qlinear(ia, s, ca, iw, r, cw, inp["K"])
    assert torch.equal(a, b)
