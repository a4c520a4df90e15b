"""Shared helpers of the GPU parity tests: moving the seeded arrays to the
device and comparing the library's results with the oracle's.

Acceptance rules (OrbitQuant page, Method, read with the stated tolerances):
  * codebook indices equal the oracle's except where the oracle's u lies
    within 1e-6 (N(0,1) units) of a decision threshold, and the fraction of
    mismatches stays below 1e-5 -- checked against the plain fp64 decision
    and against the float32 decision the kernels take;
  * stored bf16 row norms equal the oracle's fp64 norm rounded to bf16,
    except where that norm lies within 1e-6 relative of a bf16 rounding
    midpoint (then either neighbour is accepted);
  * per-group fp16 scales (int8/int4) likewise at fp16 midpoints, and the
    integer codes equal round-half-even(w'/scale) under the scale the GPU
    chose, except within 1.5e-6 * qmax of a half-integer: the kernels'
    float32 w' is within ~1e-6 of the group's largest |w'| (measured), i.e.
    within 1e-6 * qmax in units of the scale.
"""
import numpy as np
import torch

import oracle

BAND = 1e-6           # decision band in N(0,1) units around each threshold
MAX_FLIP_FRAC = 1e-5  # allowed fraction of index mismatches (all inside the band)
OUT_TOL = 2e-3        # relative Frobenius error of layer outputs on the same codes
TIE_REL = 1e-6        # relative distance to a rounding midpoint that counts as a tie
CODE_TIE = 1.5e-6     # half-integer band of w'/scale for group codes, times qmax


def to_dev(a, device="cuda"):
    """fp32 arrays stay fp32; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def as_f64(a):
    a = np.asarray(a)
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def bits_of(t):
    """A device bf16/fp16 tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_indices(gpu_packed, bits, d, u_ref, thresholds, what=""):
    """GPU indices equal the oracle's except inside the decision band, for
    both the fp64 decision (the plain definition) and the float32 one.
    Returns (stats, unpacked GPU indices); stats hold the mismatch counts of
    both decisions and the fraction of coordinates inside the band."""
    got = oracle.unpack_indices(gpu_packed.cpu().numpy() if hasattr(gpu_packed, "cpu")
                                else gpu_packed, bits, d)
    near = oracle.boundary_band(u_ref, thresholds, BAND)
    finite = np.isfinite(u_ref)
    stats = dict(n=int(got.size), band=float(near[finite].mean()) if finite.any() else 0.0)
    for decision in ("f64", "f32"):
        ref = oracle.quantize_codes(u_ref, thresholds, decision)
        bad = got != ref
        outside = bad & ~near & finite
        assert not outside.any(), (
            f"{what} ({decision} decision): {int(outside.sum())} index mismatches outside "
            f"the band, first at {np.argwhere(outside)[:5].tolist()}")
        frac = float(bad[finite].mean()) if finite.any() else 0.0
        assert frac < MAX_FLIP_FRAC, f"{what} ({decision} decision): mismatch fraction {frac}"
        stats[f"mismatch_{decision}"] = int(bad[finite].sum())
        stats[f"frac_{decision}"] = frac
    return stats, got


def _round_neighbours(x, to_bits, from_bits):
    """The two rounded values around the interval x (1 -+ TIE_REL)."""
    lo = from_bits(to_bits(x * (1 - TIE_REL)))
    hi = from_bits(to_bits(x * (1 + TIE_REL)))
    return lo, hi


def check_bf16_norms(got_bits, r64, what=""):
    """Stored bf16 norms: bit-exact against bf16_RNE(fp64 norm), except at a
    verified tie, where the GPU value must be one of the two neighbours."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    r64 = np.asarray(r64, dtype=np.float64)
    want = oracle.f64_to_bf16_bits(r64)
    bad = got_bits != want
    if bad.any():
        lo, hi = _round_neighbours(r64[bad], oracle.f64_to_bf16_bits, oracle.bf16_bits_to_f64)
        got = oracle.bf16_bits_to_f64(got_bits[bad])
        assert np.all(lo != hi), (f"{what}: {int((lo == hi).sum())} bf16 norms differ off a "
                                  f"rounding tie, first rows {np.nonzero(bad)[0][:5].tolist()}")
        assert np.all((got == lo) | (got == hi)), f"{what}: bf16 norm is neither neighbour"
    return int(bad.sum())


def check_group_codes(got_q, got_scale_bits, wrot, group, qmax, what=""):
    """Per-group symmetric codes (int8: qmax 127, int4: qmax 7).

    Scales: bit-exact against fp16_RNE(max|w'| / qmax) from the fp64 w',
    except at a verified fp16 tie (then either neighbour).  Codes: equal to
    clamp(round_half_even(w' / scale), -qmax, qmax) under the scale the GPU
    chose, except where w'/scale lies within CODE_TIE * qmax of a
    half-integer (fp32 w' errors move a tie either way).  Returns the
    mismatch counts."""
    N, d = wrot.shape
    G = wrot.reshape(N, d // group, group)
    amax = np.max(np.abs(G), axis=-1)
    want = oracle.f64_to_f16_bits(amax / qmax)
    got_scale_bits = np.asarray(got_scale_bits, dtype=np.uint16)
    s_bad = got_scale_bits != want
    if s_bad.any():
        x = amax[s_bad] / qmax
        lo, hi = _round_neighbours(x, oracle.f64_to_f16_bits, oracle.f16_bits_to_f64)
        got = oracle.f16_bits_to_f64(got_scale_bits[s_bad])
        assert np.all(lo != hi), f"{what}: fp16 scale differs off a rounding tie"
        assert np.all((got == lo) | (got == hi)), f"{what}: fp16 scale is neither neighbour"
    sc = oracle.f16_bits_to_f64(got_scale_bits)[..., None]
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(sc > 0, G / sc, 0.0)
    q_ref = np.clip(np.rint(ratio), -qmax, qmax).reshape(N, d)
    bad = np.asarray(got_q, dtype=np.int64) != q_ref
    if bad.any():
        r = ratio.reshape(N, d)[bad]
        dist = np.abs(np.abs(r - np.floor(r)) - 0.5)
        assert np.all(dist <= CODE_TIE * qmax), (
            f"{what}: {int((dist > CODE_TIE * qmax).sum())} codes differ off a half-integer tie")
    assert bad.mean() < 1e-4, f"{what}: code mismatch fraction {bad.mean()}"
    return dict(scale_mismatches=int(s_bad.sum()), code_mismatches=int(bad.sum()))


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def out_f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(bits_of(t))
    return t.detach().cpu().numpy().astype(np.float64)
