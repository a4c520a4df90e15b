"""Pins for the oracle's int4 rotated weight-only path (CPU only)."""
import os

import numpy as np

import oracle
from oracle import int4
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_hand.txt")


def _small(N=24, K=512, M=16):
    inp = synth.make(3, M=M, N=N, K=K)
    W = synth.bf16_bits_to_f32(inp["W"]).astype(np.float64)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    return inp, W, X


def test_hand_example():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        w, sbits, q, packed = [f.strip() for f in line.split("|")]
        w = np.array([[float(v) for v in w.split()]])
        n = w.shape[1]
        want_q = [int(v) for v in q.split()]
        want_bytes = [int(v, 16) for v in packed.split()]
        for decision in ("f32", "f64"):
            p = int4.int4_pack(w, np.arange(n), np.ones(n, np.int8), 1, group=n, decision=decision)
            assert int(p["scale_f16"][0, 0]) == int(sbits, 16)
            assert list(p["q"][0]) == want_q
        assert list(int4.pack_nibbles(np.array([want_q]))[0]) == want_bytes
        assert list(int4.unpack_nibbles(np.array([want_bytes], np.uint8), n)[0]) == want_q


def test_nibbles_round_trip_every_code():
    # every code in [-8, 7] at both nibble positions
    codes = np.arange(-8, 8)
    q = np.stack(np.meshgrid(codes, codes, indexing="ij"), -1).reshape(1, -1)
    p = int4.pack_nibbles(q)
    assert p.shape == (1, q.shape[1] // 2)
    # byte value = low code mod 16 + 16 * (high code mod 16)
    assert np.array_equal(p[0].astype(np.int64), (q[0, 0::2] % 16) + 16 * (q[0, 1::2] % 16))
    assert np.array_equal(int4.unpack_nibbles(p, q.shape[1]), q.astype(np.int8))


def test_codes_are_nearest_grid_points():
    """Brute force: q is the integer in [-7, 7] nearest to w'/scale (ties to
    even), decided in float32 like the kernels."""
    inp, W, _ = _small(N=6, K=256)
    p = int4.int4_pack(W, inp["perm"], inp["signs"], inp["h"], 128)
    g = oracle.f64_to_f32(p["wrot"]).reshape(6, 2, 128)
    sc = oracle.f16_bits_to_f64(p["scale_f16"]).astype(np.float32)
    ratio = (g / sc[..., None]).astype(np.float64)
    cand = np.arange(-7, 8, dtype=np.float64)
    dist = np.abs(ratio[..., None] - cand)
    best = dist.min(-1, keepdims=True)
    ties = np.sum(dist == best, -1) > 1
    q = p["q"].reshape(6, 2, 128).astype(np.float64)
    pick = cand[np.argmin(dist, -1)]
    assert np.array_equal(q[~ties], pick[~ties])
    assert np.all(q[ties] % 2 == 0)


def test_rounding_error_bound_and_range():
    inp, W, _ = _small()
    p = int4.int4_pack(W, inp["perm"], inp["signs"], inp["h"], 128)
    q = p["q"].astype(np.float64)
    sc = oracle.f16_bits_to_f64(p["scale_f16"])
    err = np.abs(int4.int4_dequant(p["q"], p["scale_f16"]) - p["wrot"]).reshape(W.shape[0], -1, 128)
    assert np.all(err <= sc[..., None] * (0.5 + 1e-5))
    assert np.all(np.abs(q) <= 7)
    # fp16 rounding of max|w'|/7 moves the largest ratio by < 0.01: it rounds to 7
    assert np.all(np.max(np.abs(q).reshape(W.shape[0], -1, 128), axis=-1) == 7)


def test_grid_weights_round_trip_exactly():
    """Weights whose rotated rows lie on the grid come back exactly."""
    rng = np.random.default_rng(5)
    N, K, h = 8, 256, 64
    perm, signs = synth.rotation_params(K, 11)
    q0 = rng.integers(-7, 8, size=(N, K))
    q0[:, ::128] = 7                                     # every group reaches 7
    sc = 2.0 ** rng.integers(-9, -3, size=(N, K // 128))  # fp16-exact scales
    wrot = (q0.reshape(N, -1, 128) * sc[..., None]).reshape(N, K)
    W = oracle.rpbh_inverse_rotate(wrot, perm, signs, h)
    p = int4.int4_pack(W, perm, signs, h, 128)
    assert np.array_equal(p["q"], q0.astype(np.int8))
    assert np.array_equal(oracle.f16_bits_to_f64(p["scale_f16"]), sc)


def test_error_is_preserved_by_inverse_rotation():
    inp, W, X = _small()
    p = int4.int4_pack(W, inp["perm"], inp["signs"], inp["h"], 128)
    y, W_hat = int4.int4_linear(X, p["q"], p["scale_f16"], inp["perm"], inp["signs"], inp["h"])
    deq = int4.int4_dequant(p["q"], p["scale_f16"])
    assert abs(np.linalg.norm(W_hat - W) - np.linalg.norm(deq - p["wrot"])) < 1e-12 * np.linalg.norm(W)
    Xrot = oracle.rpbh_rotate(X, inp["perm"], inp["signs"], inp["h"])
    y2 = int4.int4_linear_rotated(Xrot, p["q"], p["scale_f16"])
    assert np.linalg.norm(y - y2) / np.linalg.norm(y) < 1e-12
    # a dense product with the explicit matrix gives the same layer
    Pi = oracle.rpbh_matrix(inp["perm"], inp["signs"], inp["h"])
    y3 = X @ (deq @ Pi).T
    assert np.linalg.norm(y - y3) / np.linalg.norm(y) < 1e-12
    # 4-bit: coarser than int8, still a usable layer
    ref = X @ W.T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 0.2


def test_zero_group_and_tiny_scales():
    n = 256
    W = np.zeros((3, n))
    W[1, :128] = 1.0
    # max/7 = 7.1e-8 rounds to the smallest fp16 subnormal 2^-24 = 5.96e-8:
    # the ratio 8.4 clamps to 7
    W[2, :128] = 5e-7
    ident = np.arange(n), np.ones(n, np.int8)
    p = int4.int4_pack(W, *ident, 1, 128)
    assert np.all(p["q"][0] == 0) and np.all(p["scale_f16"][0] == 0)
    assert np.all(p["q"][1, 128:] == 0) and p["scale_f16"][1, 1] == 0
    assert p["scale_f16"][2, 0] == 1 and np.all(p["q"][2, :128] == 7)
