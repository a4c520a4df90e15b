"""Shared helpers of the GPU parity tests: moving the seeded arrays to the
device and comparing the library's results with the oracle's."""
import numpy as np
import torch

import oracle

BAND = 1e-6           # decision band in N(0,1) units around each threshold
MAX_FLIP_FRAC = 1e-5  # allowed fraction of index mismatches (all inside the band)
OUT_TOL = 2e-3        # relative Frobenius error of layer outputs on the same codes


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
    """GPU indices equal the oracle's except inside the decision band."""
    got = oracle.unpack_indices(gpu_packed.cpu().numpy(), bits, d)
    ref = oracle.quantize_codes(u_ref, thresholds, "f32")
    bad = got != ref
    near = oracle.boundary_band(u_ref, thresholds, BAND)
    finite = np.isfinite(u_ref)
    outside = bad & ~near & finite
    assert not outside.any(), (
        f"{what}: {int(outside.sum())} index mismatches outside the band, "
        f"first at {np.argwhere(outside)[:5].tolist()}")
    frac = bad[finite].mean() if finite.any() else 0.0
    assert frac < MAX_FLIP_FRAC, f"{what}: mismatch fraction {frac}"
    return dict(mismatches=int(bad.sum()), band=float(near.mean()), n=int(bad.size)), got


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def out_f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(bits_of(t))
    return t.detach().cpu().numpy().astype(np.float64)
