"""Pins for the oracle's quantizer, packing and layer product (CPU only)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing.txt")


@pytest.mark.parametrize("K", [4, 16, 64])
def test_threshold_count_is_nearest_centroid(K):
    cb = oracle.lloyd_max_gaussian(K)
    u = np.random.default_rng(K).standard_normal(200000) * 1.3
    far = ~oracle.boundary_band(u, cb["thresholds"], 1e-9)
    idx = oracle.quantize_codes(u, cb["thresholds"], "f64")
    nearest = np.argmin(np.abs(u[:, None] - cb["centroids"][None, :]), axis=1)
    np.testing.assert_array_equal(idx[far], nearest[far])


def test_ties_go_to_the_lower_cell():
    cb = oracle.lloyd_max_gaussian(16)
    t = cb["thresholds"]
    assert oracle.quantize_codes(np.array([0.0]), t, "f64")[0] == 7
    assert oracle.quantize_codes(np.array([-0.0]), t, "f64")[0] == 7
    assert list(oracle.quantize_codes(t, t, "f64")) == list(range(15))
    assert oracle.quantize_codes(np.array([-50.0, 50.0]), t)[0] == 0
    assert oracle.quantize_codes(np.array([-50.0, 50.0]), t)[1] == 15


def test_f32_decision_rounds_before_comparing():
    t = np.array([1.0])
    u = np.array([1.0 + 2.0 ** -30])       # above 1 in fp64, equal to 1 in fp32
    assert oracle.quantize_codes(u, t, "f64")[0] == 1
    assert oracle.quantize_codes(u, t, "f32")[0] == 0


def _golden_packing():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        b, idx, byts = [f.strip() for f in line.split("|")]
        yield int(b), [int(v) for v in idx.split()], [int(v, 16) for v in byts.split()]


@pytest.mark.parametrize("case", list(_golden_packing()), ids=lambda c: f"b{c[0]}-{c[1]}")
def test_packing_hand_examples(case):
    bits, idx, byts = case
    got = oracle.pack_indices(np.array([idx]), bits)[0]
    assert list(got) == byts
    assert list(oracle.unpack_indices(got[None], bits, len(idx))[0]) == idx


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_pack_round_trip(bits):
    n = 96
    idx = np.random.default_rng(bits).integers(0, 2 ** bits, size=(5, n))
    p = oracle.pack_indices(idx, bits)
    assert p.shape == (5, n * bits // 8)
    np.testing.assert_array_equal(oracle.unpack_indices(p, bits, n), idx)


def test_qlinear_codes_matches_triple_loop():
    g = np.random.default_rng(3)
    M, N, d = 3, 4, 8
    ca, cw = oracle.codebook(4)["centroids"], oracle.codebook(2)["centroids"]
    ia, iw = g.integers(0, 16, (M, d)), g.integers(0, 4, (N, d))
    s = g.random(M) * 10
    r_bits = oracle.f64_to_bf16_bits(g.random(N) * 3)
    bias = g.standard_normal(N)
    y = oracle.qlinear_codes(ia, s, ca, iw, r_bits, cw, d, bias)
    r = oracle.bf16_bits_to_f64(r_bits)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(d):
                acc += (ca[ia[m, k]] / np.sqrt(d)) * (cw[iw[n, k]] / np.sqrt(d))
            assert abs(r[n] * s[m] * acc + bias[n] - y[m, n]) < 1e-12 * (1 + abs(y[m, n]))


def test_unquantized_factorisation_is_exact():
    # with the quantizer removed, r s <w~, x~> = W x (eps = 0)
    inp = synth.make(1)
    W, X = inp["W"].astype(np.float64), inp["X"].astype(np.float64)
    y = oracle.qlinear_unquantized(X, W, inp["perm"], inp["signs"], inp["h"])
    ref = X @ W.T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-12


def test_activation_norm_is_token_norm_and_error_matches_distortion():
    inp = synth.make(2, M=64, N=8)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    cb = oracle.codebook(4)
    q = oracle.quant_act(X, inp["perm"], inp["signs"], inp["h"], cb, 4, synth.EPS)
    np.testing.assert_allclose(q["s"], np.linalg.norm(X, axis=1), rtol=1e-13)
    # On Gaussian tokens every rotated coordinate of the unit direction is
    # ~N(0, 1/d), so the mean squared error of the quantized direction is the
    # codebook's distortion D.  (Tokens whose energy sits in a few outlier
    # channels keep uneven block energies after the rotation and land above D.)
    inp = synth.make(3, M=256, N=8)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    d = X.shape[1]
    for bits in (2, 4):
        cb = oracle.codebook(bits)
        q = oracle.quant_act(X, inp["perm"], inp["signs"], inp["h"], cb, bits, synth.EPS)
        xt = q["xrot"] / (q["s"][:, None] + synth.EPS)
        err = np.sum((cb["centroids"][q["idx"]] / np.sqrt(d) - xt) ** 2, axis=1)
        assert abs(np.mean(err) / cb["distortion"] - 1) < 0.03


def test_weight_pack_norms_and_zero_row():
    inp = synth.make(1, N=16)
    W = inp["W"].astype(np.float64)
    W[5] = 0.0
    cb = oracle.codebook(4)
    p = oracle.pack_weights(W, inp["perm"], inp["signs"], inp["h"], cb, 4)
    np.testing.assert_allclose(p["r"], np.linalg.norm(W, axis=1), rtol=1e-13)
    assert p["r_bf16"][5] == 0 and np.all(p["idx"][5] == 7)
    r_back = oracle.bf16_bits_to_f64(p["r_bf16"])
    np.testing.assert_allclose(r_back, p["r"], rtol=2 ** -8)


def test_whole_layer_error_is_small_and_decreases_with_bits():
    # the quantized layer approximates W x (OrbitQuant: W^' x^' ~ W x); the
    # relative error shrinks as the codebooks get finer
    inp = synth.make(2, M=64, N=64)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    W = synth.bf16_bits_to_f32(inp["W"]).astype(np.float64)
    ref = X @ W.T
    errs = []
    for bits in (2, 4, 6):
        cb = oracle.codebook(bits)
        a = oracle.quant_act(X, inp["perm"], inp["signs"], inp["h"], cb, bits, synth.EPS)
        w = oracle.pack_weights(W, inp["perm"], inp["signs"], inp["h"], cb, bits)
        y = oracle.qlinear_codes(a["idx"], a["s"], cb["centroids"], w["idx"], w["r_bf16"],
                                 cb["centroids"], X.shape[1])
        errs.append(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    assert errs[0] > errs[1] > errs[2]
    # W4A4 on these tokens: about sqrt(D_w + D_a) ~ 0.14, more with outliers
    assert errs[1] < 0.25


def test_gelu_matches_torch():
    x = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu_erf(x), ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
