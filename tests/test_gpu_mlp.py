"""The DiT MLP pair (up 3072 -> 12288, GELU, down 12288 -> 3072, W2A4) with
the activation fused into the up layer's GEMM epilogue and the down layer's
permutation folded into the up layer's weight rows.

OrbitQuant page, Method: the down layer quantizes Pi_down x with
Pi_down = blkdiag(H D) P_pi.  GELU acts elementwise, so P_pi GELU(z) =
GELU(P_pi z): permuting the up layer's output rows by pi (its weight rows,
norms and bias) hands the down layer activations that are already in
permuted order, and the down layer's rotation keeps only blkdiag(H D) (the
identity permutation).  Checks: the GELU epilogue against the oracle on the
same codes, and the fold as exact identities of the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import OUT_TOL, bits_of, out_f64, rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _oracle_gelu_out(ia, s, iw, r, ba, bw, K, bias=None):
    A = oracle.unpack_indices(ia.cpu().numpy(), ba, K)
    B = oracle.unpack_indices(iw.cpu().numpy(), bw, K)
    y = oracle.qlinear_codes(A, s.cpu().numpy(), oracle.codebook(ba)["centroids"], B,
                             bits_of(r), oracle.codebook(bw)["centroids"], K, bias)
    return oracle.gelu_erf(y)


@pytest.mark.parametrize("M,N,K,odt", [(1024, 2048, 512, torch.bfloat16),   # full 128x128 tiles
                                       (77, 130, 256, torch.float32),       # ragged tiles
                                       (300, 200, 256, torch.bfloat16)])
def test_qlinear_gelu_epilogue(gpu_lib, M, N, K, odt):
    rbp = gpu_lib
    inp = synth.make(4, M=M, N=N, K=K, h=128)
    rot = rbp.Rotation(inp["perm"], inp["signs"], 128)
    ca, cw = rbp.Codebook(K, 4), rbp.Codebook(K, 2)
    ia, s = rbp.quant_act(rot, ca, to_dev(inp["X"]), synth.EPS)
    iw, r = rbp.pack_weights(rot, cw, to_dev(inp["W"]))
    bias = torch.from_numpy(np.random.default_rng(M).standard_normal(N).astype(np.float32)).cuda()
    out = rbp.qlinear(ia, s, ca, iw, r, cw, K, bias=bias, out_dtype=odt, act="gelu")
    ref = _oracle_gelu_out(ia, s, iw, r, 4, 2, K, bias.cpu().numpy())
    assert rel_fro(out_f64(out), ref) < OUT_TOL


def test_mlp_pair_fold_is_exact(gpu_lib):
    rbp = gpu_lib
    M, K, N = 256, 512, 1024                       # up: K -> N, down: N -> K
    inp = synth.make(4, M=M, N=N, K=K, h=128)
    perm2, signs2 = synth.rotation_params(N, 77)   # the down layer's rotation
    X = to_dev(inp["X"])
    W_up = inp["W"]                                # [N, K]
    rot_up = rbp.Rotation(inp["perm"], inp["signs"], 128)
    ca, cw = rbp.Codebook(K, 4), rbp.Codebook(K, 2)
    ia, s = rbp.quant_act(rot_up, ca, X, synth.EPS)
    bias = torch.from_numpy(np.random.default_rng(1).standard_normal(N).astype(np.float32)).cuda()

    # plain: up layer in natural order, GELU in the epilogue
    iw, r = rbp.pack_weights(rot_up, cw, to_dev(W_up))
    H = rbp.qlinear(ia, s, ca, iw, r, cw, K, bias=bias, act="gelu")
    # folded: weight rows (and bias) in the down layer's gather order
    iw_f, r_f = rbp.pack_weights(rot_up, cw, to_dev(np.ascontiguousarray(W_up[perm2])))
    H_f = rbp.qlinear(ia, s, ca, iw_f, r_f, cw, K, bias=bias[torch.from_numpy(perm2).long().cuda()],
                      act="gelu")
    torch.cuda.synchronize()
    p = torch.from_numpy(perm2).long().cuda()
    assert torch.equal(H_f.view(torch.int16), H[:, p].contiguous().view(torch.int16))

    # down layer: full RPBH on H == identity permutation on the folded H_f
    ca2 = rbp.Codebook(N, 4)
    rot_down = rbp.Rotation(perm2, signs2, 256)
    rot_down_f = rbp.Rotation(np.arange(N, dtype=np.int32), signs2, 256)
    i1, s1 = rbp.quant_act(rot_down, ca2, H, synth.EPS)
    i2, s2 = rbp.quant_act(rot_down_f, ca2, H_f, synth.EPS)
    torch.cuda.synchronize()
    # the norm is summed from the rows in memory order, so the folded rows
    # round differently in the last bits; codes may differ only where that
    # moves u across a threshold
    s1, s2 = s1.cpu().numpy().astype(np.float64), s2.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s1 - s2) <= 1e-6 * s1)
    a1 = oracle.unpack_indices(i1.cpu().numpy(), 4, N)
    a2 = oracle.unpack_indices(i2.cpu().numpy(), 4, N)
    assert np.mean(a1 != a2) <= 1e-5
