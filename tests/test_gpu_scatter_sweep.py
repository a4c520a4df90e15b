"""A seeded sweep of the activation quantizer over row widths, block sizes,
code widths and row counts, on random permuting rotations: the scatter form
(the rotation's plan) and the gather form (no plan) must agree bit for bit,
and sampled rows' codes must equal the oracle's outside the 1e-6 decision
band (OrbitQuant page, Method: x' = Pi x, u = sqrt(d) x' / (s + eps),
idx = #{t_j < u}).  The mismatch fraction bar is checked on the large
samples of the other tests; a sample of a few rows holds too few codes for
it (with 255 thresholds one in-band tie can exceed it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import BAND, as_f64, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        h = int(rng.choice([128, 256]))
        d = int(rng.choice([1024, 2048, 3072, 4096, 8192, 12288, 16384]))
        bits = int(rng.choice([2, 3, 4, 6, 8] if h == 256 else [2, 4, 6, 8]))
        M = int(rng.integers(1, 5000 if d <= 4096 else 1500))
        out.append((d, h, bits, M, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("d,h,bits,M,seed", _cases())
def test_scatter_sweep(gpu_lib, d, h, bits, M, seed):
    rbp = gpu_lib
    rng = np.random.default_rng(seed)
    perm = rng.permutation(d).astype(np.int32)
    signs = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    scale = np.exp(rng.normal(0.0, 1.0, (M, 1)))          # a spread of token norms
    X = synth.f32_to_bf16_bits((rng.standard_normal((M, d)) * scale).astype(np.float32))
    if M > 3:
        X[M // 2] = 0                                     # a zero token
    Xd = to_dev(X)
    cb = rbp.Codebook(d, bits)
    i1, s1 = rbp.quant_act(rbp.Rotation(perm, signs, h), cb, Xd, synth.EPS)
    i2, s2 = rbp.quant_act(rbp.Rotation(perm, signs, h, plan=False), cb, Xd, synth.EPS)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 8), replace=False), [0, M - 1]]))
    ref_cb = oracle.codebook(bits)
    ref = oracle.quant_act(as_f64(X[rows]), perm, signs, h, ref_cb, bits, synth.EPS)
    got = oracle.unpack_indices(i1[rows].cpu().numpy(), bits, d)
    near = oracle.boundary_band(ref["u"], ref_cb["thresholds"], BAND)
    for decision in ("f64", "f32"):
        bad = got != oracle.quantize_codes(ref["u"], ref_cb["thresholds"], decision)
        assert not (bad & ~near).any(), f"{decision}: {int((bad & ~near).sum())} mismatches outside the band"
    s_ref = np.linalg.norm(as_f64(X), axis=1)
    assert np.all(np.abs(s1.cpu().numpy().astype(np.float64) - s_ref) <= 1e-6 * s_ref)
