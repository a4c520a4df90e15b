"""fp64 CPU oracle of the rotate-then-quantize linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The library (``rotation_bit_ptq_amd``) never imports this package and this
package imports nothing from the library: the two share no code, tables or
constants.  Inputs come from ``synth`` (random draws only).

It is written as a plain, slow, direct reading of the pages, in float64:

* OrbitQuant paper page (hyper.ai, "OrbitQuant"), section Method:
  the RPBH rotation Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi, the
  offline weight rotation W' = W Pi^T with row norms r' kept in BF16 and unit
  directions quantized by one Lloyd-Max codebook fitted to the fixed marginal
  f_d ~ N(0, 1/d); the online activation rotation x' = Pi x, split into
  s = ||x'|| and x' / (s + eps), quantized by the same kind of codebook; and
  the product W^' x^' ~ W x with no inverse rotation.
* Int8 rotated-weight article (cloud.baidu.com, "量化旋转压缩主模型技术解析",
  section 4 "How it works"): rotate -> per-group scale -> round -> store;
  at load time dequantize -> inverse-rotate -> ordinary layer forward.
  Its 4-bit sibling (``int4``) stands for the INT4 projections the OrbitQuant
  page's Experiments section favours in its ablations.

Readings where the pages are silent:
Hadamard matrices are Sylvester-ordered and orthonormal (H_h / sqrt(h));
P_pi gathers, (P_pi x)_k = x[pi(k)]; the signs D act on the permuted index;
the codebook is stored in N(0,1) units (the N(0,1/d) codebook is it divided
by sqrt(d)); the quantizer returns idx = #{j : t_j < u} for the sorted
midpoint thresholds t_j; index k of a row takes bits [k*b, (k+1)*b) of the
row's LSB-first byte stream; int8 uses the symmetric range [-127, 127], a
per-(row, group of 128) fp16 scale fp16(max|w'| / 127) and round half to even;
int4 is the same recipe with [-7, 7] and fp16(max|w'| / 7), codes stored as
two's-complement nibbles, low nibble first.

Where a floating-point value decides an integer (a codebook index, a bf16 row
norm, an fp16 scale, an int8 code), the decision is taken in float32, the
precision of the HIP kernels, from the fp64 value (``decision="f32"``);
``decision="f64"`` takes it in float64 for reference.

Pins (tests/test_oracle_*.py): every function here is checked against
something other than itself -- closed forms, library routines on special
cases, textbook Lloyd-Max tables (tests/golden/), brute force on tiny
inputs, and invariants of the mathematics.  Parity unpinned: none of the
whole-layer numbers -- the pages print no worked example, test vector or
layer-level value, so end-to-end outputs are pinned only through the
invariants above.
"""
from .numfmt import (bf16_bits_to_f64, f64_to_bf16_bits, f16_bits_to_f64,
                     f64_to_f16_bits, f64_to_f32)
from .hadamard import sylvester, fwht
from .rotation import (rpbh_matrix, rpbh_rotate, rpbh_inverse_rotate,
                       block_rht_rotate, full_rht_rotate, haar_matrix)
from .codebook import (lloyd_max_gaussian, codebook, lloyd_max_sphere, codebook_sphere,
                       sphere_distortion)
from .orbit import (quantize_codes, boundary_band, pack_indices, unpack_indices,
                    pack_weights, quant_act, qlinear_codes, qlinear_unquantized,
                    gelu_erf)
from .int8 import int8_pack, int8_dequant, int8_linear
from .int4 import int4_pack, int4_dequant, int4_linear, pack_nibbles, unpack_nibbles

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "f16_bits_to_f64", "f64_to_f16_bits",
    "f64_to_f32", "sylvester", "fwht", "rpbh_matrix", "rpbh_rotate",
    "rpbh_inverse_rotate", "block_rht_rotate", "full_rht_rotate", "haar_matrix",
    "lloyd_max_gaussian", "codebook", "lloyd_max_sphere", "codebook_sphere",
    "sphere_distortion", "quantize_codes", "boundary_band",
    "pack_indices", "unpack_indices", "pack_weights", "quant_act",
    "qlinear_codes", "qlinear_unquantized", "gelu_erf", "int8_pack",
    "int8_dequant", "int8_linear", "int4_pack", "int4_dequant", "int4_linear",
    "pack_nibbles", "unpack_nibbles",
]
