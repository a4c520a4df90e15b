"""Pins for the oracle's int8 rotated weight-only path (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from oracle.int8 import int8_linear_rotated
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int8_hand.txt")


def _small(N=24, K=512, M=16):
    inp = synth.make(3, M=M, N=N, K=K)
    W = synth.bf16_bits_to_f32(inp["W"]).astype(np.float64)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    return inp, W, X


def test_hand_example():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        w, sbits, q = [f.strip() for f in line.split("|")]
        w = np.array([[float(v) for v in w.split()]])
        n = w.shape[1]
        for decision in ("f32", "f64"):
            p = oracle.int8_pack(w, np.arange(n), np.ones(n, np.int8), 1, group=n,
                                 decision=decision)
            assert int(p["scale_f16"][0, 0]) == int(sbits, 16)
            assert list(p["q"][0]) == [int(v) for v in q.split()]


def test_rounding_error_bound_and_range():
    inp, W, _ = _small()
    p = oracle.int8_pack(W, inp["perm"], inp["signs"], inp["h"], 128)
    q, wrot = p["q"].astype(np.float64), p["wrot"]
    sc = oracle.f16_bits_to_f64(p["scale_f16"])
    deq = oracle.int8_dequant(p["q"], p["scale_f16"], 128)
    err = np.abs(deq - wrot).reshape(W.shape[0], -1, 128)
    # |w^' - w'| <= scale/2 (float32 decision adds at most a few float32 ulps)
    assert np.all(err <= sc[..., None] * (0.5 + 1e-5))
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.max(np.abs(q).reshape(W.shape[0], -1, 128), axis=-1) == 127)


def test_error_is_preserved_by_inverse_rotation():
    inp, W, X = _small()
    p = oracle.int8_pack(W, inp["perm"], inp["signs"], inp["h"], 128)
    y, W_hat = oracle.int8_linear(X, p["q"], p["scale_f16"], inp["perm"], inp["signs"], inp["h"])
    deq = oracle.int8_dequant(p["q"], p["scale_f16"])
    # orthogonality: ||W^ - W||_F = ||W^' - W'||_F
    assert abs(np.linalg.norm(W_hat - W) - np.linalg.norm(deq - p["wrot"])) < 1e-12 * np.linalg.norm(W)
    # dequant -> inverse rotate -> X W^T equals (X Pi^T) W^'^T
    Xrot = oracle.rpbh_rotate(X, inp["perm"], inp["signs"], inp["h"])
    y2 = int8_linear_rotated(Xrot, p["q"], p["scale_f16"])
    assert np.linalg.norm(y - y2) / np.linalg.norm(y) < 1e-12
    # and the whole int8 layer is close to the bf16 layer
    ref = X @ W.T
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 2e-2


def test_f32_and_f64_decisions_agree_off_ties():
    inp, W, _ = _small(N=64)
    a = oracle.int8_pack(W, inp["perm"], inp["signs"], inp["h"], 128, "f32")
    b = oracle.int8_pack(W, inp["perm"], inp["signs"], inp["h"], 128, "f64")
    assert np.mean(a["scale_f16"] != b["scale_f16"]) < 1e-3
    assert np.mean(a["q"] != b["q"]) < 1e-4


def test_zero_group():
    n = 256
    W = np.zeros((2, n))
    W[1, :128] = 1.0
    p = oracle.int8_pack(W, np.arange(n), np.ones(n, np.int8), 1, 128)
    assert np.all(p["q"][0] == 0) and np.all(p["scale_f16"][0] == 0)
    assert np.all(p["q"][1, 128:] == 0) and p["scale_f16"][1, 1] == 0
