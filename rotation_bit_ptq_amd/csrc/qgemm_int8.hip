// Int8 and int4 weight-only GEMM kernels on rotated fp16 activations (see
// qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
namespace {

// Narrow batches (M <= 32 tokens, e.g. conditioning vectors, where the
// slab-walking kernel below does not apply): the product is bound by the
// weight stream.  Each workgroup owns 32 weight rows and all
// tokens; its WV waves split K in groups of 128 (one scale group), reduced
// in LDS.  Per group a lane reads whole cache lines: 64 (int8) or 32 (int4)
// contiguous bytes of its weight row (the two halves of a row are adjacent)
// and 128 contiguous bytes of each token row; the MFMA k order inside the
// group is k = 64 half + 8 s + j for both operands (s = 0..7).  Each wave
// keeps P groups in flight, and the sub-steps alternate between two
// accumulators.  The MFMA's second operand holds the tokens (MB blocks of
// 32; rows past M re-read row M - 1 and are dropped).
template <class OpB, int MB, int WV, int P>
__global__ __launch_bounds__(512) void narrow_kernel(GemmArgs g) {
  constexpr int kWBytes = 64 * OpB::kCodeBits / 8;  // weight bytes per lane per group
  constexpr int kWVec = kWBytes / 16;
  __shared__ float red[WV > 1 ? WV - 1 : 1][MB][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const long long n0 = (long long)blockIdx.x * 32;
  const long long nr = n0 + r32 < g.N ? n0 + r32 : g.N - 1;
  const uint32_t ob = (uint32_t)(nr * g.ldb) + (uint32_t)(half * kWBytes);
  const uint16_t* const srow = g.scale_f16 + nr * g.groups_per_row;
  uint32_t oa[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const long long m = 32 * mb + r32 < g.M ? 32 * mb + r32 : g.M - 1;
    oa[mb] = (uint32_t)(m * g.lda) + (uint32_t)(half * 128);
  }
  const int per = g.groups_per_row / WV;  // groups of this wave
  const int c0 = wave * per, c1 = c0 + per, cm = c0 + (per / P) * P;

  floatx16 acc[2][MB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[s][mb][q] = 0.0f;
  u32x4 wt[P][kWVec];
  u32x4 tk[P][MB][8];
  uint32_t sc[P];
  auto load = [&](int slot, int c) {
    c = c < c1 ? c : c1 - 1;  // past the end: re-read the last group (unused)
#pragma unroll
    for (int v = 0; v < kWVec; ++v) wt[slot][v] = *(const u32x4*)(g.b + ob + (uint32_t)c * (2u * kWBytes) + 16u * v);
    const uint32_t s16 = srow[c];
    sc[slot] = s16 | (s16 << 16);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 8; ++v) tk[slot][mb][v] = *(const u32x4*)(g.a + oa[mb] + (uint32_t)c * 256u + 16u * v);
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      OpB op;
      op.scale2 = sc[slot];
      half8 bv;
      if constexpr (OpB::kCodeBits == 8) {
        const u32x4 w = wt[slot][s >> 1];
        op.v = w;
        bv = op.decode(s & 1, 0);
      } else {
        const u32x4 w = wt[slot][s >> 2];
        const uint32_t d = (s & 3) == 0 ? w.x : (s & 3) == 1 ? w.y : (s & 3) == 2 ? w.z : w.w;
        op.v = make_uint2(d, 0u);
        bv = op.decode(0, 0);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[s & 1][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            bv, __builtin_bit_cast(half8, tk[slot][mb][s]), acc[s & 1][mb], 0, 0, 0);
    }
  };
  // whole rounds of P groups through the ring, then the remaining groups one
  // at a time
#pragma unroll
  for (int p = 0; p < P; ++p) load(p, c0 + p);
  for (int c = c0; c < cm; c += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      compute(p);
      load(p, c + p + P);
    }
  }
  for (int c = cm; c < c1; ++c) {
    load(0, c);
    compute(0);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[0][mb] += acc[1][mb];
  if (wave > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[wave - 1][mb][q][lane] = acc[0][mb][q];
  }
  __syncthreads();
  if (wave != 0) return;
  // lane l, element q of token block mb: weight row n0 + 8 (q / 4) + 4 half
  // + q % 4, token 32 mb + r32
  const bool f32_out = g.out_dtype != ORBIT_BF16;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const long long m = 32 * mb + r32;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const long long n = n0 + 8 * (q / 4) + 4 * half + (q % 4);
      float y = acc[0][mb][q];
#pragma unroll
      for (int w = 0; w < WV - 1; ++w) y += red[w][mb][q][lane];
      if (m < g.M && n < g.N) {
        const float v = y + load_bias(g, n);
        if (f32_out) ((float*)g.out)[m * g.N + n] = v;
        else ((uint16_t*)g.out)[m * g.N + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Batches of at most 16 tokens with 8 G scale groups per row (G <= 4):
// the weight stream is the whole cost, so the kernel is laid out for memory
// parallelism at low register cost.  One workgroup of eight waves per
// compute unit; wave w owns the G groups G w .. G w + G - 1 of every row and
// keeps the tokens of those groups in registers for the whole launch.  The workgroup walks 16-row weight slabs
// blockIdx.x, blockIdx.x + gridDim.x, ..., with the weights of three slabs
// in flight per wave, multiplying each with v_mfma_f32_16x16x32_f16 (the
// weights as the 16-row operand, the tokens as the 16-column operand, so no
// token row is loaded twice).  Per group and lane: 32 k of one weight row
// (32 bytes of int8 or 16 of int4) and 32 k of one token row (64 bytes),
// k = 128 group + 32 (lane / 16) + 8 s + j for MFMA s = 0..3 and j < 8 on
// both operands.  Each wave's partial sums of a slab go to LDS; after the
// walk, wave w adds the eight partials of slabs w, w + 8, ... and writes
// them.  Tokens past M re-read token M - 1 and weight rows past N re-read
// row N - 1; neither is written.
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <class OpB, int G>
__global__ __launch_bounds__(512) void narrow16_kernel(GemmArgs g, int slabs_per_block) {
  constexpr int WV = 8, P = 3;
  constexpr bool kI4 = OpB::kCodeBits == 4;
  constexpr int kWVec = kI4 ? 1 : 2;                 // 16-byte weight loads per lane and group
  constexpr uint32_t kGroupBytes = kI4 ? 64u : 128u;  // weight bytes of one row and group
  extern __shared__ __align__(16) char smem[];
  floatx4* const red = (floatx4*)smem;  // [slab of the block][wave][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const long long slabs = (g.N + 15) / 16;
  const int g0 = wave * G;

  u32x4 tk[G][4];
  {
    const long long m = r16 < g.M ? r16 : g.M - 1;
    const uint8_t* src = g.a + m * g.lda + (uint32_t)kq * 64u;
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) tk[q][v] = *(const u32x4*)(src + (uint32_t)(g0 + q) * 256u + 16u * v);
  }
  u32x4 wt[P][G][kWVec];
  uint32_t sc[P][G];
  auto slab_of = [&](int i) { return (long long)blockIdx.x + (long long)i * gridDim.x; };
  auto load = [&](int slot, int i) {
    const long long n0 = slab_of(i) * 16 + r16;
    const long long n = n0 < g.N ? n0 : g.N - 1;
    const uint8_t* src = g.b + n * g.ldb + (uint32_t)kq * (kGroupBytes / 4u);
#pragma unroll
    for (int q = 0; q < G; ++q) {
#pragma unroll
      for (int v = 0; v < kWVec; ++v) wt[slot][q][v] = *(const u32x4*)(src + (uint32_t)(g0 + q) * kGroupBytes + 16u * v);
      const uint32_t s16 = g.scale_f16[n * g.groups_per_row + g0 + q];
      sc[slot][q] = s16 | (s16 << 16);
    }
  };
  auto compute = [&](int slot) {
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        OpB op;
        op.scale2 = sc[slot][q];
        half8 bv;
        if constexpr (kI4) {
          op.v = make_uint2(wt[slot][q][0][s], 0u);
          bv = op.decode(0, 0);
        } else {
          op.v = wt[slot][q][s >> 1];
          bv = op.decode(s & 1, 0);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv, __builtin_bit_cast(half8, tk[q][s]), acc, 0, 0, 0);
      }
    return acc;
  };
  // Slab i of the block is valid while blockIdx.x + i gridDim.x < slabs
  // (the same for every wave); invalid slabs are neither loaded nor
  // computed.
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (slab_of(p) < slabs) load(p, p);
  __builtin_amdgcn_sched_barrier(0);
  for (int i0 = 0; i0 < slabs_per_block; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = i0 + p;
      if (i < slabs_per_block && slab_of(i) < slabs) {
        red[(i * WV + wave) * 64 + lane] = compute(p);
        if (slab_of(i + P) < slabs) load(p, i + P);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  // lane l holds weight rows 16 slab + 4 (l / 16) + 0..3 of token l % 16
  const bool f32_out = g.out_dtype != ORBIT_BF16;
  for (int i = wave; i < slabs_per_block && slab_of(i) < slabs; i += WV) {
    floatx4 y = red[(i * WV) * 64 + lane];
#pragma unroll
    for (int w = 1; w < WV; ++w) y += red[(i * WV + w) * 64 + lane];
    const long long m = r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const long long n = slab_of(i) * 16 + 4 * kq + r;
      if (m < g.M && n < g.N) {
        const float v = y[r] + load_bias(g, n);
        if (f32_out) ((float*)g.out)[m * g.N + n] = v;
        else ((uint16_t*)g.out)[m * g.N + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Up to 16 tokens and 8, 16, 24 or 32 groups per row: the slab-walking
// kernel, one workgroup per compute unit (more when a workgroup would own
// more than eight slabs, which bounds its LDS to 64 KB).
template <class OpB>
hipError_t launch_narrow16(GemmArgs& g, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const long long slabs = (g.N + 15) / 16;
  long long blocks = slabs < di.n_cu ? slabs : di.n_cu;
  if ((slabs + blocks - 1) / blocks > 8) blocks = (slabs + 7) / 8;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int per = (int)((slabs + blocks - 1) / blocks);
  const size_t lds = (size_t)per * 8 * 64 * 16;
  switch (g.groups_per_row) {
    case 8:
      hipLaunchKernelGGL((narrow16_kernel<OpB, 1>), dim3((unsigned)blocks), dim3(512), lds, stream, g, per);
      break;
    case 16:
      hipLaunchKernelGGL((narrow16_kernel<OpB, 2>), dim3((unsigned)blocks), dim3(512), lds, stream, g, per);
      break;
    case 24:
      hipLaunchKernelGGL((narrow16_kernel<OpB, 3>), dim3((unsigned)blocks), dim3(512), lds, stream, g, per);
      break;
    case 32:
      hipLaunchKernelGGL((narrow16_kernel<OpB, 4>), dim3((unsigned)blocks), dim3(512), lds, stream, g, per);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Eight waves split K when it holds a multiple of eight groups, four when a
// multiple of four, else one.
template <class OpB, int MB>
hipError_t launch_narrow(GemmArgs& g, hipStream_t stream) {
  const long long blocks = (g.N + 31) / 32;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (g.groups_per_row % 8 == 0)
    hipLaunchKernelGGL((narrow_kernel<OpB, MB, 8, 2>), dim3((unsigned)blocks), dim3(512), 0, stream, g);
  else if (g.groups_per_row % 4 == 0)
    hipLaunchKernelGGL((narrow_kernel<OpB, MB, 4, 2>), dim3((unsigned)blocks), dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((narrow_kernel<OpB, MB, 1, 2>), dim3((unsigned)blocks), dim3(64), 0, stream, g);
  return hipGetLastError();
}

// Up to 16 tokens with 8, 16, 24 or 32 groups per row take the slab-walking
// kernel, other batches of up to 32 tokens the 32-row narrow kernel; large
// products the LDS-staged kernel (256 x 256 tiles, a ring of three 64-k
// chunks); the rest the register-fed kernel and its smaller tiles.  The staged kernel reads each
// fp16 group scale through the aligned dword that holds it, so it also needs
// a 4-byte aligned scale array with an even number of entries (else the last
// dword would reach past the array).
template <class OpB>
hipError_t launch_weight_only(GemmArgs& g, hipStream_t stream) {
  if (g.M <= 16 && g.groups_per_row % 8 == 0 && g.groups_per_row <= 32) return launch_narrow16<OpB>(g, stream);
  if (g.M <= 32) return launch_narrow<OpB, 1>(g, stream);
  const long long tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
  const bool scales_ok = ((uintptr_t)g.scale_f16 & 3) == 0 && (g.N * g.groups_per_row) % 2 == 0;
  if (tiles >= 128 && scales_ok) {
    constexpr int kStage = 256 * 64 * 2 + 256 * 64 * OpB::kCodeBits / 8 + 256 * 4;
    return launch_tile<2, F16Op, OpB, 8, 2>(g, 3 * kStage, stream);
  }
  return launch_shape<1, F16Op, OpB>(g, 0, stream);
}

}  // namespace

hipError_t launch_int8(GemmArgs& g, hipStream_t stream) { return launch_weight_only<I8Op>(g, stream); }
hipError_t launch_int4(GemmArgs& g, hipStream_t stream) { return launch_weight_only<I4Op>(g, stream); }
}  // namespace qgemm
}  // namespace orbit
