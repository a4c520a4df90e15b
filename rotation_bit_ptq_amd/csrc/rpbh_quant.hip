// Host entry of the row kernels (rotate, rotate + quantize, int8 pack): fills
// the kernel arguments and dispatches on input type and mode.  The kernels
// are in rpbh_impl.h, instantiated in the rpbh_*.hip files.
#include <cmath>

#include "rpbh_impl.h"
#include "rpbh_mfma2.h"

namespace orbit {

hipError_t launch_rows(const RowJob& job, hipStream_t stream) {
  using namespace rows;
  RowArgs a = {};
  a.d = job.d;
  a.h = job.h;
  a.log2h = 0;
  while ((1 << a.log2h) < job.h) ++a.log2h;
  a.nslots = job.d / kSlot;
  a.nrounds = (a.nslots + kWave - 1) / kWave;
  a.rows = job.rows;
  a.perm = job.perm;
  a.sign_bits = job.sign_bits;
  a.gather = nullptr;  // set below when the plan's order is the kernel's
  a.perm_identity = job.perm_identity ? 1 : 0;
  a.in = job.in;
  a.sqrt_d_over_h = (float)sqrt((double)job.d / job.h);
  a.sqrt_h_over_d = (float)sqrt((double)job.h / job.d);
  a.inv_sqrt_h = (float)(1.0 / sqrt((double)job.h));
  a.inv_h = (float)(1.0 / job.h);
  a.eps = job.eps;
  a.ga = job.grid.a;
  a.gb = job.grid.b;
  a.cells = job.grid.cells;
  a.nthr = job.grid.nthr;
  a.grid_bias = 0xA8000000u;
  for (int i = 0; i < job.grid.nthr && job.thresholds; ++i) a.thr[i] = job.thresholds[i];
  // small grids are built here with the kernels' float32 cell function
  if (job.thresholds && job.grid.cells <= kArgCells) {
    a.cells_in_args = 1;
    for (int c = 0; c < job.grid.cells; ++c) {
      a.cell_t[c] = INFINITY;
      a.cell_base[c] = 0;
    }
    const float top = kMagic + (float)(job.grid.cells - 1);
    for (int j = 0; j < job.grid.nthr; ++j) {
      float f = std::fmaf(job.thresholds[j], job.grid.a, job.grid.b);
      f = std::fmin(std::fmax(f, kMagic), top);
      const int cj = (int)(f - kMagic);
      a.cell_t[cj] = job.thresholds[j];
      for (int c = cj + 1; c < job.grid.cells; ++c) a.cell_base[c] += 1;
    }
  }
  a.idx_out = job.idx_out;
  a.s_out = job.norm_f32_out;
  a.r_out = job.norm_bf16_out;
  a.xrot_f32 = job.xrot_f32_out;
  a.xrot_f16 = (uint16_t*)job.rot_out;
  a.group = job.group;
  a.q_out = job.q_out;
  a.scale_out = job.scale_out;
  const bool quant = job.mode == RowMode::kActQuant || job.mode == RowMode::kWeightQuant;
  a.grid_bytes = quant ? job.grid.cells * (int)sizeof(GridCell) : 0;
  const int esz = job.in_dtype == ORBIT_BF16 ? 2 : 4;
  a.row_bytes = 2 * job.d * esz;
  a.wave_bytes = a.row_bytes;
  if (job.rows == 0) return hipSuccess;
  const bool bf16 = job.in_dtype == ORBIT_BF16;
  // bf16 rows with h = 64, 128 or 256: transposed-gather kernels
  const bool tr_order = job.h == 64 || job.h == 128 || job.h == 256;
  const bool fast = bf16 && tr_order && (!quant || job.bits != 1);
  // the gather plan serves the kernels whose gather order it was built in
  // (transposed exactly when h allows it)
  if (job.gather && fast == tr_order) a.gather = job.gather;
  const uint32_t* words = job.gather && mfma_words_len(job.d, job.h) > 0
                              ? (const uint32_t*)(job.gather + gather_len(job.d)) : nullptr;
  // the scatter section serves permuting rotations (an identity permutation
  // reads the padded row in place, without bank conflicts)
  const uint32_t* scatter = job.gather && !job.perm_identity && scatter_len(job.d, job.h) > 0
      ? (const uint32_t*)(job.gather + gather_len(job.d) + mfma_words_len(job.d, job.h)) : nullptr;
  const bool rot_f16 = job.mode == RowMode::kRotate && job.out_dtype == ORBIT_F16;
  // blocks of 512 .. 4096 coordinates on rows of 2048 or 4096 (the full
  // RHT): the h = 128 factor on the matrix cores, the block bits above it
  // in registers and across lanes (rpbh_mfma2.h, big_kernel)
  if (bf16 && ((quant && m2_big_takes(job.d, job.h, job.bits, false)) ||
               (rot_f16 && m2_big_takes(job.d, job.h, 0, true)))) {
    a.mfma_words = words;
    if (rot_f16) return launch_m2_big<kRotF16>(a, 0, stream);
    return job.mode == RowMode::kActQuant ? launch_m2_big<kAct>(a, job.bits, stream)
                                          : launch_m2_big<kWeight>(a, job.bits, stream);
  }
  // bf16 rows with h = 128 or 256 and d = 1024 .. 4096 (one wave per row) or
  // 8192, 12288, 16384 (four waves per row): the Hadamard runs on the
  // matrix cores and each lane packs and stores its own runs of codes
  // (rpbh_mfma2.h), reading the plan's offset words in that kernel's order
  // when the rotation has a plan.
  if (bf16 && ((quant && m2_takes(job.d, job.h, job.bits, false)) ||
               (rot_f16 && m2_takes(job.d, job.h, 0, true)))) {
    a.mfma_words = words;
    a.scatter_words = scatter;
    const bool act = job.mode == RowMode::kActQuant;
    if (job.h == 128) {
      if (rot_f16) return launch_m2<kRotF16, 4>(a, 0, stream);
      return act ? launch_m2<kAct, 4>(a, job.bits, stream) : launch_m2<kWeight, 4>(a, job.bits, stream);
    }
    if (rot_f16) return launch_m2<kRotF16, 8>(a, 0, stream);
    return act ? launch_m2<kAct, 8>(a, job.bits, stream) : launch_m2<kWeight, 8>(a, job.bits, stream);
  }
  // The first matrix-core kernels (rpbh_mfma.h) stage codes in LDS: h = 64,
  // and 3-bit codes with h = 128.  The plan's words are in their order only
  // for h = 64; otherwise they build their offsets from pi and the signs.
  a.mfma_words = job.h == 64 ? words : nullptr;
  const bool mfma = fast && quant &&
                    ((job.d % 1024 == 0 && job.d <= 4096) || job.d == 8192 || job.d == 12288 || job.d == 16384);
  const bool mfma_rot = fast && rot_f16 && job.d % 1024 == 0 && job.d <= 4096;
  if (mfma_rot) {
    if (job.h == 64) return launch_mfma<kRotF16, 2>(a, 0, stream);
    if (job.h == 128) return launch_mfma<kRotF16, 4>(a, 0, stream);
    return launch_mfma<kRotF16, 8>(a, 0, stream);
  }
  if (mfma) {
    const bool act = job.mode == RowMode::kActQuant;
    if (job.h == 64) return act ? launch_mfma<kAct, 2>(a, job.bits, stream) : launch_mfma<kWeight, 2>(a, job.bits, stream);
    if (job.h == 128) return act ? launch_mfma<kAct, 4>(a, job.bits, stream) : launch_mfma<kWeight, 4>(a, job.bits, stream);
    return act ? launch_mfma<kAct, 8>(a, job.bits, stream) : launch_mfma<kWeight, 8>(a, job.bits, stream);
  }
  if (fast) {
    const int lt = job.h == 64 ? 2 : (job.h == 128 ? 3 : 4);
    if (job.mode == RowMode::kActQuant) {
      if (lt == 2) return launch_fast<kAct, 2>(a, job.bits, stream);
      if (lt == 3) return launch_fast<kAct, 3>(a, job.bits, stream);
      return launch_fast<kAct, 4>(a, job.bits, stream);
    }
    if (job.mode == RowMode::kWeightQuant) {
      if (lt == 2) return launch_fast<kWeight, 2>(a, job.bits, stream);
      if (lt == 3) return launch_fast<kWeight, 3>(a, job.bits, stream);
      return launch_fast<kWeight, 4>(a, job.bits, stream);
    }
    if (job.mode == RowMode::kInt8Pack) {
      if (lt == 2) return launch_fast<kInt8, 2>(a, 0, stream);
      if (lt == 3) return launch_fast<kInt8, 3>(a, 0, stream);
      return launch_fast<kInt8, 4>(a, 0, stream);
    }
    if (job.mode == RowMode::kInt4Pack) {
      if (lt == 2) return launch_fast<kInt4, 2>(a, 0, stream);
      if (lt == 3) return launch_fast<kInt4, 3>(a, 0, stream);
      return launch_fast<kInt4, 4>(a, 0, stream);
    }
    if (job.out_dtype == ORBIT_F16) {
      if (lt == 2) return launch_fast<kRotF16, 2>(a, 0, stream);
      if (lt == 3) return launch_fast<kRotF16, 3>(a, 0, stream);
      return launch_fast<kRotF16, 4>(a, 0, stream);
    }
    if (lt == 2) return launch_fast<kRotF32, 2>(a, 0, stream);
    if (lt == 3) return launch_fast<kRotF32, 3>(a, 0, stream);
    return launch_fast<kRotF32, 4>(a, 0, stream);
  }
  switch (job.mode) {
    case RowMode::kActQuant:
      return bf16 ? launch_mode<uint16_t, kAct>(a, job.bits, stream)
                  : launch_mode<float, kAct>(a, job.bits, stream);
    case RowMode::kWeightQuant:
      return bf16 ? launch_mode<uint16_t, kWeight>(a, job.bits, stream)
                  : launch_mode<float, kWeight>(a, job.bits, stream);
    case RowMode::kRotate:
      if (job.out_dtype == ORBIT_F16)
        return bf16 ? launch_mode<uint16_t, kRotF16>(a, 0, stream)
                    : launch_mode<float, kRotF16>(a, 0, stream);
      return bf16 ? launch_mode<uint16_t, kRotF32>(a, 0, stream)
                  : launch_mode<float, kRotF32>(a, 0, stream);
    case RowMode::kInt8Pack:
      return bf16 ? launch_mode<uint16_t, kInt8>(a, 0, stream)
                  : launch_mode<float, kInt8>(a, 0, stream);
    case RowMode::kInt4Pack:
      return bf16 ? launch_mode<uint16_t, kInt4>(a, 0, stream)
                  : launch_mode<float, kInt4>(a, 0, stream);
  }
  return hipErrorInvalidValue;
}

// Gather plan: entry r*1024 + l*16 + e = element offset (in the x, -x row
// buffer) of the coordinate lane l gathers as element e of round r.
template <int LT>
__global__ __launch_bounds__(256) void gather_plan_kernel(int d, const int32_t* perm,
                                                          const uint32_t* sign_bits, uint16_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= gather_len(d)) return;
  const int r = i >> 10, l = (i >> 4) & 63, e = i & 15;
  const int slot = r * rows::kWave + l;
  uint32_t v = 0;
  if (slot < d / rows::kSlot) {
    int k = slot * rows::kSlot + e;
    if constexpr (LT >= 0) k = rows::tr_k<LT>(slot, e);
    const uint32_t neg = (sign_bits[k >> 5] >> (k & 31)) & 1u;
    v = (uint32_t)perm[k] + neg * (uint32_t)d;
  }
  out[i] = (uint16_t)v;
}

// The plan's matrix-core section, in the order of the kernel that reads it.
// h = 64 (rpbh_mfma.h): word 4 (64 c + l) + q serves lane l of pair c
// (positions 512 c .. + 511), element pair 2 q, 2 q + 1 of the lane's
// fragment, i.e. permuted coordinates k and k + 1 with k = 512 c + 32 (l %
// 16) + 8 (l / 16) + 2 q: byte offsets 2 pi(k) and 2 pi(k + 1) of the
// unpadded row in the low and high halves, their sign flips in bits 15 and
// 31.  h = 128 .. 4096 (rpbh_mfma2.h): word 4 (64 o + l) + q serves lane l
// of A operand o, slots 2 q and 2 q + 1 (m2::slot_k, in the h = 256 order
// for h = 256 and in the h = 128 order otherwise), with the byte offsets of
// that kernel's row layout (padded up to 12288 coordinates).
__global__ __launch_bounds__(256) void mfma_words_kernel(int d, int h, const int32_t* perm,
                                                         const uint32_t* sign_bits, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d / 2) return;
  const int o = i >> 8, l = (i >> 2) & 63, q = i & 3;
  int k0, k1;
  uint32_t a0, a1;
  if (h == 64) {
    k0 = 512 * o + 32 * (l & 15) + 8 * (l >> 4) + 2 * q;
    k1 = k0 + 1;
    a0 = (uint32_t)perm[k0] * 2u;
    a1 = (uint32_t)perm[k1] * 2u;
  } else {
    const int kq = l >> 4, r16 = l & 15;
    k0 = h != 256 ? rows::m2::slot_k<4>(o, kq, r16, 2 * q) : rows::m2::slot_k<8>(o, kq, r16, 2 * q);
    k1 = h != 256 ? rows::m2::slot_k<4>(o, kq, r16, 2 * q + 1) : rows::m2::slot_k<8>(o, kq, r16, 2 * q + 1);
    const bool pad = rows::m2::padded(d);
    a0 = pad ? rows::m2::row_addr<true>(perm[k0]) : rows::m2::row_addr<false>(perm[k0]);
    a1 = pad ? rows::m2::row_addr<true>(perm[k1]) : rows::m2::row_addr<false>(perm[k1]);
  }
  const uint32_t s0 = (sign_bits[k0 >> 5] >> (k0 & 31)) & 1u;
  const uint32_t s1 = (sign_bits[k1 >> 5] >> (k1 & 31)) & 1u;
  out[i] = a0 | (s0 << 15) | (a1 << 16) | (s1 << 31);
}

// The plan's scatter section (h = 128 / 256 packed-code kernels): entry
// pi(k) holds the byte offset 16 (64 o + l) + 2 j of slot j of lane l in A
// operand o, the slot whose permuted coordinate is k (the inverse of
// m2::slot_k), and D_k in bit 15.  A lane that loaded x[i] writes it,
// sign-flipped, to that offset: the operands then lie in LDS as 16
// contiguous bytes per lane.
__global__ __launch_bounds__(256) void scatter_words_kernel(int d, int h, const int32_t* perm,
                                                            const uint32_t* sign_bits, uint16_t* out) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= d) return;
  int o, kq, r16, j;
  if (h == 128) {  // k = 512 o + 128 (r16 / 4) + 32 kq + 4 j + r16 % 4
    o = k >> 9;
    kq = (k >> 5) & 3;
    j = (k >> 2) & 7;
    r16 = 4 * ((k >> 7) & 3) + (k & 3);
  } else {         // k = 1024 (o / 2) + 256 (r16 / 4) + 64 kq + 8 j + 4 (o % 2) + r16 % 4
    o = 2 * (k >> 10) + ((k >> 2) & 1);
    kq = (k >> 6) & 3;
    j = (k >> 3) & 7;
    r16 = 4 * ((k >> 8) & 3) + (k & 3);
  }
  const uint32_t off = 16u * (uint32_t)(64 * o + 16 * kq + r16) + 2u * (uint32_t)j;
  const uint32_t neg = (sign_bits[k >> 5] >> (k & 31)) & 1u;
  out[perm[k]] = (uint16_t)(off | (neg << 15));
}

hipError_t launch_gather_plan(int d, int h, const int32_t* perm, const uint32_t* sign_bits,
                              uint16_t* out, hipStream_t stream) {
  if (mfma_words_len(d, h) > 0)
    hipLaunchKernelGGL(mfma_words_kernel, dim3((d / 2 + 255) / 256), dim3(256), 0, stream, d, h, perm,
                       sign_bits, (uint32_t*)(out + gather_len(d)));
  if (scatter_len(d, h) > 0)
    hipLaunchKernelGGL(scatter_words_kernel, dim3((d + 255) / 256), dim3(256), 0, stream, d, h, perm,
                       sign_bits, out + gather_len(d) + mfma_words_len(d, h));
  const dim3 grid(gather_len(d) / 256), block(256);
  if (h == 64) hipLaunchKernelGGL(gather_plan_kernel<2>, grid, block, 0, stream, d, perm, sign_bits, out);
  else if (h == 128) hipLaunchKernelGGL(gather_plan_kernel<3>, grid, block, 0, stream, d, perm, sign_bits, out);
  else if (h == 256) hipLaunchKernelGGL(gather_plan_kernel<4>, grid, block, 0, stream, d, perm, sign_bits, out);
  else hipLaunchKernelGGL(gather_plan_kernel<-1>, grid, block, 0, stream, d, perm, sign_bits, out);
  return hipGetLastError();
}

}  // namespace orbit
