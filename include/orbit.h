/*
 * orbit.h -- C ABI of the rotate-then-quantize linear layer for AMD MI355X
 * (gfx950).  Library: liborbit.so (rotation_bit_ptq_amd/liborbit.so).
 *
 * The method (OrbitQuant paper page on hyper.ai, section Method):
 *   offline  W' = W Pi_d^T; row norms r'_i = ||w'_i|| stored in BF16; unit
 *            rows quantized by one Lloyd-Max codebook C_d.
 *   online   x' = Pi_d x; s = ||x'||; x' / (s + eps) quantized by C_d.
 *   product  out[m, n] = r_n s_m <Q(w~_n), Q(x~_m)>  ~  (W x_m)_n,
 *            with no inverse rotation at run time.
 *   Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi  (the RPBH rotation).
 * And the int8 rotated weight-only path of the int8 article (cloud.baidu.com,
 * "量化旋转压缩主模型技术解析", section 4): rotate, per-group scale, round;
 * at run time dequantize and undo the rotation (computed here in the equal
 * form (X Pi^T) (W^')^T, so the weights are never inverse-rotated).
 *
 * Conventions shared by every entry point
 *   - Readings of the pages: (P_pi x)_k = x[perm[k]] (gather); sign bit k
 *     applies to permuted coordinate k; H_h is Sylvester-ordered and scaled
 *     by 1/sqrt(h), so Pi_d is orthogonal.
 *   - Codebooks are in N(0,1) units: coordinate v of a unit vector in
 *     dimension d is coded as idx = #{j : thresholds[j] < sqrt(d) * v} and
 *     decodes to centroids[idx] / sqrt(d).  The decision is taken in float32.
 *   - Packed indices: row-major, one LSB-first bit stream per row; index k
 *     takes bits [k*bits, (k+1)*bits); a row of d indices is d*bits/8 bytes.
 *   - Ownership: the caller owns every buffer.  Pointers named "device" are
 *     HIP device memory; structs passed by pointer are host memory read only
 *     during the call.  The library allocates no device memory and keeps no
 *     state between calls; every entry point is thread-safe.
 *   - Asynchrony: device work is enqueued on `stream` (0 = the default
 *     stream) and the call returns without synchronizing.  Buffers must not
 *     alias.
 *   - Errors: no entry point throws or aborts.  Arguments are validated on
 *     the host before any HIP call; a bad argument returns ORBIT_E_ARG
 *     (null pointer, bad enum, unsorted codebook), ORBIT_E_SHAPE (sizes) or
 *     ORBIT_E_DTYPE, with nothing enqueued.  A failed launch returns
 *     ORBIT_E_HIP and orbit_last_hip_error reports the HIP code.
 */
#ifndef ORBIT_H
#define ORBIT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORBIT_OK = 0,
  ORBIT_E_ARG = 1,
  ORBIT_E_SHAPE = 2,
  ORBIT_E_DTYPE = 3,
  ORBIT_E_UNSUPPORTED = 4,
  ORBIT_E_HIP = 5
} orbit_status;

typedef enum { ORBIT_F32 = 0, ORBIT_BF16 = 1, ORBIT_F16 = 2 } orbit_dtype;

/* RPBH rotation parameters (the int8 article's "rotation metadata").
 * d: dimension, a multiple of h, 16 <= d <= ORBIT_MAX_D.
 * h: Hadamard block size, a power of two, 16 <= h <= 1024, or 2048 / 4096
 *    when d <= 4096.
 * perm: device int32[d], a permutation of 0..d-1 (gather order).
 * sign_bits: device uint32[(d + 31) / 32]; bit k%32 of word k/32 set means
 *            D_k = -1 for permuted coordinate k.
 * Variants of the rotation ablation (OrbitQuant page, Experiments): an
 * identity perm gives Block-RHT, h = d gives the full RHT (d a power of two
 * up to 4096). */
typedef struct {
  int32_t d;
  int32_t h;
  const int32_t *perm;
  const uint32_t *sign_bits;
  /* Optional (NULL allowed): the rotation's gather plan, built by
   * orbit_rpbh_build_gather for this perm, sign_bits, d and h; device,
   * 16-byte aligned, orbit_rpbh_gather_len(d, h) entries.  With it the
   * row kernels read each lane's gather offsets directly instead of
   * deriving them from perm and sign_bits in every workgroup. */
  const uint16_t *gather;
  /* Set by orbit_rpbh_build_gather, not by the caller:
   * ORBIT_RPBH_IDENTITY when it found perm[k] == k for every k (Block-RHT,
   * or a permutation folded into the producer of the rows), which lets the
   * matrix-core kernels read each fragment as contiguous bytes instead of
   * gathering it; 0 otherwise.  The entry points honour the bit only
   * together with a gather plan (gather != NULL); without one it is ignored
   * and the rows are gathered through perm. */
  int32_t flags;
} orbit_rpbh;

#define ORBIT_RPBH_IDENTITY 1

#define ORBIT_MAX_D 16384
#define ORBIT_MAX_LEVELS 256

/* Lloyd-Max codebook in N(0,1) units (OrbitQuant page, Method: one
 * codebook per input dimension d, fitted offline to the fixed marginal
 * f_d ~ N(0, 1/d); by scale equivariance that is the N(0,1) codebook divided
 * by sqrt(d)).  Levels = 2^bits.  centroids ascending and symmetric;
 * thresholds[j] = (centroids[j] + centroids[j+1]) / 2, the middle one 0. */
typedef struct {
  int32_t bits; /* 1, 2, 3, 4, 6 or 8 */
  int32_t d;    /* dimension it serves (informational; the table is d-free) */
  float centroids[ORBIT_MAX_LEVELS];
  float thresholds[ORBIT_MAX_LEVELS - 1];
} orbit_codebook;

/* Text of a status code (static storage). */
const char *orbit_status_string(orbit_status status);

/* Writes to *hip_error_out the HIP error code of the last call on this
 * thread that returned ORBIT_E_HIP (0 if none has).  Host only.
 * Errors: ORBIT_E_ARG (hip_error_out NULL). */
orbit_status orbit_last_hip_error(int *hip_error_out);

/* Length in uint16 entries of the gather plan of a rotation of dimension d
 * and block h: 1024 per round of 1024 coordinates, at least 4096
 * (L = 1024 * max(4, ceil(d / 1024))), plus d entries of matrix-core words
 * when h is 64 .. 4096 and d is a multiple of 512 (d <= 16384), plus d
 * entries of the scatter section when h is 128 or 256 and d is 1024, 2048,
 * 3072, 4096, 8192, 12288 or 16384; 0 for invalid d, h.  Host only. */
int64_t orbit_rpbh_gather_len(int32_t d, int32_t h);

/* Builds the gather plan of `rot` (its `gather` field is ignored) into the
 * device buffer `out` of orbit_rpbh_gather_len(d, h) entries, 16-byte
 * aligned, on `stream`, and sets rot->flags: it reads perm back to the host
 * once (so the call synchronizes `stream`) and sets ORBIT_RPBH_IDENTITY
 * exactly when perm is the identity.  Entry r*1024 + l*16 + e is the
 * offset, in elements of the row buffer that holds x followed by -x, of the
 * coordinate y_k = D_k x[perm[k]] (OrbitQuant page, Method: P_pi then the
 * signs) that lane l gathers as element e of round r, i.e.
 * perm[k] + (D_k = -1 ? d : 0), and 0 past the end of the row.  With
 * s = 64 r + l: k = 16 s + e in general; for h = 64, 128 and 256 (T = h/16
 * lanes per Hadamard block, G = 16/T, p = s mod T, e = G t + i) the order
 * that applies H_h = H_T x H_16 as H_T first: k = 16 (s - p) + 16 t + G p + i.
 * The matrix-core section (when present) follows at entry L as uint32 words
 * in the order of the kernel that reads it; each word covers two permuted
 * coordinates k0, k1 as off(k0) | (D_k0 = -1) << 15 | off(k1) << 16 |
 * (D_k1 = -1) << 31, off(k) the byte offset of x[perm[k]] in that kernel's
 * LDS copy of the row.  h = 64: word 4 (64 c + l) + q, k0 = 512 c +
 * 32 (l mod 16) + 8 floor(l / 16) + 2 q, k1 = k0 + 1, off(k) = 2 perm[k].
 * h = 128 .. 4096: word 4 (64 o + l) + q holds slots j = 2 q, 2 q + 1 of
 * A operand o of lane l = 16 kq + r16, slot j being coordinate
 * 512 o + 128 floor(r16 / 4) + 32 kq + 4 j + (r16 mod 4) for h != 256 and
 * 1024 floor(o / 2) + 256 floor(r16 / 4) + 64 kq + 8 j + 4 (o mod 2) +
 * (r16 mod 4) for h = 256; off(k) = 2 p + 16 floor(p / 64) with p = perm[k]
 * when d <= 12288 (a 16-byte pad after every 64 coordinates), 2 p beyond.
 * The scatter section (when present) follows the words: d uint16 entries,
 * entry perm[k] = off'(k) | (D_k = -1) << 15, off'(k) = 16 (64 o + l) + 2 j
 * for the slot (o, l, j) of the h = 128 / 256 order above that holds
 * coordinate k: the LDS byte offset at which the activation quantizer's
 * lanes write x[perm[k]], sign-flipped, so that each lane's operand is 16
 * contiguous bytes.
 * Errors: ORBIT_E_ARG (null or misaligned pointers, or perm not a
 * permutation of 0 .. d-1), ORBIT_E_SHAPE (d, h), ORBIT_E_HIP. */
orbit_status orbit_rpbh_build_gather(orbit_rpbh *rot, uint16_t *out, hipStream_t stream);

/* Fit the Lloyd-Max codebook for N(0,1) with 2^bits levels, in fp64, on the
 * host (OrbitQuant page, Method: Lloyd-Max run offline on the marginal).
 * Alternates the nearest-neighbour and centroid conditions, then polishes
 * with Newton steps on the thresholds until the step is below `tol`
 * (<= 0 selects 1e-15) or `max_iter` Newton steps (<= 0 selects 100).
 * out: receives the float32 tables (required).  centroids_f64[2^bits],
 * thresholds_f64[2^bits - 1] and mse_f64 (the distortion E[(X - Q(X))^2])
 * are optional host outputs (may be NULL).  No device work.
 * Errors: ORBIT_E_ARG (bits not in {1,2,3,4,6,8}, out NULL, d < 1). */
orbit_status orbit_fit_codebook(int32_t d, int32_t bits, int32_t max_iter, double tol,
                                orbit_codebook *out, double *centroids_f64,
                                double *thresholds_f64, double *mse_f64);

/* Lloyd-Max codebook on the exact marginal f_d (OrbitQuant page, Method):
 * one coordinate T of a direction uniform on the unit sphere S^{d-1}, with
 * density proportional to (1 - t^2)^((d-3)/2), in N(0,1) units u = sqrt(d) t
 * (so |u| <= sqrt(d) and E[u^2] = 1).  As d grows it tends to the N(0,1)
 * codebook of orbit_fit_codebook; for d = 3 it is the uniform quantizer of
 * [-sqrt 3, sqrt 3].  Arguments, outputs and method as orbit_fit_codebook.
 * Errors: ORBIT_E_ARG (bits not in {1,2,3,4,6,8}, out NULL, d < 3),
 * ORBIT_E_UNSUPPORTED (no ordered fixed point reached). */
orbit_status orbit_fit_codebook_sphere(int32_t d, int32_t bits, int32_t max_iter, double tol,
                                       orbit_codebook *out, double *centroids_f64,
                                       double *thresholds_f64, double *mse_f64);

/* Offline weight packer (OrbitQuant page, Method, offline stage):
 * W' = W Pi^T row by row, r_n = ||w'_n|| rounded to bf16 (nearest even),
 * u = sqrt(d) w'_n / r_n (u = 0 for a zero row), idx = #{t_j < u}.
 * W: device [d_out, d_in] row-major, w_dtype F32 or BF16; rot->d == d_in.
 * idx_out: device uint8 [d_out, d_in * cw->bits / 8]; r_bf16_out: device
 * uint16 [d_out] (bf16 bits).  d_out >= 0 (0 enqueues nothing). */
orbit_status orbit_pack_weights(const orbit_rpbh *rot, const orbit_codebook *cw,
                                const void *W, orbit_dtype w_dtype,
                                int64_t d_out, int64_t d_in,
                                uint8_t *idx_out, uint16_t *r_bf16_out,
                                hipStream_t stream);

/* Online activation rotate + quantize (OrbitQuant page, Method, inference):
 * x' = Pi x, s = ||x'|| (fp32), u = sqrt(d) x' / (s + eps), idx = #{t_j < u}.
 * X: device [M, d] row-major, F32 or BF16.  idx_out: device uint8
 * [M, d * ca->bits / 8]; s_out: device float [M]; xrot_f32_debug: optional
 * device float [M, d] receiving x' (NULL to skip).  eps >= 0. */
orbit_status orbit_quant_act(const orbit_rpbh *rot, const orbit_codebook *ca,
                             const void *X, orbit_dtype x_dtype, int64_t M, int64_t d,
                             float eps, uint8_t *idx_out, float *s_out,
                             float *xrot_f32_debug, hipStream_t stream);

/* Codebook-decode GEMM (OrbitQuant page, Method: W^' x^' with the rotation
 * cancelled):  out[m, n] = s[m] * r[n] / K * sum_k ca[ia[m,k]] * cw[iw[n,k]]
 *              (+ bias[n]).
 * idx_a: device [M, K*ca->bits/8]; s: device float [M]; idx_w: device
 * [N, K*cw->bits/8]; r_bf16: device uint16 [N]; bias: optional device [N]
 * (F32 or BF16, bias_dtype ignored when NULL); out: device [M, N], F32 or
 * BF16 (nearest even).  The products run on fp16 matrix cores with float32
 * accumulation.  Bits: ca 2/3/4/6/8, cw 2/3/4/6/8.  K % 128 == 0,
 * 128 <= K <= 65536; M, N >= 0. */
orbit_status orbit_qlinear(const uint8_t *idx_a, const float *s, const orbit_codebook *ca,
                           const uint8_t *idx_w, const uint16_t *r_bf16,
                           const orbit_codebook *cw, const void *bias, orbit_dtype bias_dtype,
                           int64_t M, int64_t N, int64_t K, void *out, orbit_dtype out_dtype,
                           hipStream_t stream);

/* Output activation of orbit_qlinear_act. */
typedef enum { ORBIT_ACT_NONE = 0, ORBIT_ACT_GELU = 1 } orbit_act;

/* orbit_qlinear with an elementwise activation applied in fp32 to
 * s_m r_n / K * acc (+ bias) before the single rounding of the output:
 * ORBIT_ACT_GELU is the erf GELU, x/2 (1 + erf(x / sqrt 2)), the activation
 * between the two layers of a DiT MLP.  Fusing it here removes the separate
 * activation pass over the hidden activations.  Same arguments, layouts and
 * errors as orbit_qlinear, plus ORBIT_E_ARG for an unknown act. */
orbit_status orbit_qlinear_act(const uint8_t *idx_a, const float *s, const orbit_codebook *ca,
                               const uint8_t *idx_w, const uint16_t *r_bf16,
                               const orbit_codebook *cw, const void *bias, orbit_dtype bias_dtype,
                               int64_t M, int64_t N, int64_t K, void *out, orbit_dtype out_dtype,
                               orbit_act act, hipStream_t stream);

/* Rotation alone: out = Pi x per row, the online rotation x' = Pi_d x of the
 * OrbitQuant page, Method, without the norm split and the codebook.  It is
 * the int8 article's load-and-run step (section 4) in the equal form that
 * rotates the activations instead of inverse-rotating the weights, since
 * (W^' Pi) x = W^' (Pi x); the rotation ablation of the OrbitQuant page,
 * Experiments, times it for RPBH, Block-RHT and the full RHT.
 * X: device [M, d] F32 or BF16; out: device [M, d], out_dtype F32 or F16
 * (nearest even).  Errors: ORBIT_E_ARG (null or misaligned pointers),
 * ORBIT_E_SHAPE (d, h, M), ORBIT_E_DTYPE, ORBIT_E_HIP. */
orbit_status orbit_rotate(const orbit_rpbh *rot, const void *X, orbit_dtype x_dtype,
                          int64_t M, int64_t d, void *out, orbit_dtype out_dtype,
                          hipStream_t stream);

/* Int8 rotated weight packer (int8 article, section 4 pack_weight):
 * W' = W Pi^T; for each row and each group of `group` consecutive columns
 * scale = fp16(max|w'| / 127) (float32 division, nearest even);
 * q = clamp(round_half_even(w' / scale), -127, 127), q = 0 where scale = 0.
 * W: device [N, K] F32 or BF16; q_out: device int8 [N, K];
 * scale_f16_out: device uint16 [N, K/group] (fp16 bits).
 * group a multiple of 16 dividing K, group <= 1024. */
orbit_status orbit_int8_pack_weights(const orbit_rpbh *rot, const void *W, orbit_dtype w_dtype,
                                     int64_t N, int64_t K, int32_t group,
                                     int8_t *q_out, uint16_t *scale_f16_out,
                                     hipStream_t stream);

/* Int8 weight-only GEMM on rotated activations (int8 article, section 4
 * load_and_run, in the equal form that needs no inverse rotation):
 * out[m, n] = sum_k Xrot[m,k] * q[n,k] * scale[n, k/group]  (+ bias[n]).
 * Xrot: device [M, K] F16 (from orbit_rotate); q: device int8 [N, K];
 * scale_f16: device uint16 [N, K/group]; group == 128; K % 128 == 0;
 * out: device [M, N], F32 or BF16.  Weights are decoded to fp16 (q times
 * scale, one rounding) and multiplied on fp16 matrix cores, fp32 accumulate. */
orbit_status orbit_int8_linear(const void *Xrot, orbit_dtype xrot_dtype, int64_t M, int64_t K,
                               const int8_t *q, const uint16_t *scale_f16, int32_t group,
                               int64_t N, const void *bias, orbit_dtype bias_dtype,
                               void *out, orbit_dtype out_dtype, hipStream_t stream);

/* Int4 rotated weight packer: the 4-bit sibling of orbit_int8_pack_weights
 * (int8 article, section 4 pack_weight, with the INT4 projections of the
 * OrbitQuant page's Experiments section): W' = W Pi^T; per row and group of
 * `group` consecutive columns scale = fp16(max|w'| / 7) (float32 division,
 * nearest even); q = clamp(round_half_even(w' / scale), -7, 7), q = 0 where
 * scale = 0.  W: device [N, K] F32 or BF16; q_out: device uint8 [N, K/2],
 * two's-complement nibbles, code 2j in the low nibble of byte j, code 2j+1
 * in the high nibble; scale_f16_out: device uint16 [N, K/group] (fp16 bits).
 * group a multiple of 16 dividing K, group <= 1024; q_out 16-byte aligned.
 * Errors as orbit_int8_pack_weights. */
orbit_status orbit_int4_pack_weights(const orbit_rpbh *rot, const void *W, orbit_dtype w_dtype,
                                     int64_t N, int64_t K, int32_t group,
                                     uint8_t *q_out, uint16_t *scale_f16_out,
                                     hipStream_t stream);

/* Int4 weight-only GEMM on rotated activations, the 4-bit sibling of
 * orbit_int8_linear: out[m, n] = sum_k Xrot[m,k] * q[n,k] * scale[n, k/group]
 * (+ bias[n]).  Xrot: device [M, K] F16; q: device uint8 [N, K/2] in the
 * layout orbit_int4_pack_weights writes; scale_f16: device uint16
 * [N, K/group]; group == 128; K % 128 == 0; out: device [M, N], F32 or BF16.
 * Weights are decoded to fp16 (q times scale, one rounding) and multiplied
 * on fp16 matrix cores with fp32 accumulation.  Errors as orbit_int8_linear. */
orbit_status orbit_int4_linear(const void *Xrot, orbit_dtype xrot_dtype, int64_t M, int64_t K,
                               const uint8_t *q, const uint16_t *scale_f16, int32_t group,
                               int64_t N, const void *bias, orbit_dtype bias_dtype,
                               void *out, orbit_dtype out_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ORBIT_H */
