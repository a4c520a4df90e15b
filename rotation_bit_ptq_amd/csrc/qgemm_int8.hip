// Int8 and int4 weight-only GEMM kernels on rotated fp16 activations (see
// qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
namespace {

// Narrow batches (M <= 64 tokens, e.g. conditioning vectors): the product is
// bound by the weight stream and by each wave's chain of dependent steps.
// Each workgroup owns 32 weight rows and all tokens; its WV waves split K
// (partial sums reduced in LDS), each keeps P chunks of 32 k in flight in a
// register ring, and the two sub-steps of a chunk accumulate into separate
// registers so consecutive MFMAs do not wait on each other.  The MFMA's
// second operand holds the tokens (MB blocks of 32; rows past M re-read row
// M - 1 and are dropped).
template <class OpB, int MB, int WV, int P>
__global__ __launch_bounds__(512) void narrow_kernel(GemmArgs g) {
  __shared__ float red[WV - 1][MB][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const long long n0 = (long long)blockIdx.x * 32;
  const long long nr = n0 + r32 < g.N ? n0 + r32 : g.N - 1;
  const uint32_t ob = (uint32_t)(nr * g.ldb) + (uint32_t)(half * OpB::kBytes);
  const uint16_t* const srow = g.scale_f16 + nr * g.groups_per_row;
  uint32_t oa[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const long long m = 32 * mb + r32 < g.M ? 32 * mb + r32 : g.M - 1;
    oa[mb] = (uint32_t)(m * g.lda) + (uint32_t)(half * F16Op::kBytes);
  }
  const int per = (int)(g.K / 32) / WV;  // chunks of this wave
  const int c0 = wave * per, c1 = c0 + per, cm = c0 + (per / P) * P;

  floatx16 acc[2][MB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[s][mb][q] = 0.0f;
  OpB wt[P];
  F16Op tk[P][MB];
  auto load = [&](int slot, int c) {
    c = c < c1 ? c : c1 - 1;  // past the end: re-read the last chunk (unused)
    wt[slot].load(g.b + ob + (uint32_t)c * (2u * OpB::kBytes));
    const uint32_t sc = srow[(c * 32) >> 7];
    wt[slot].scale2 = sc | (sc << 16);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tk[slot][mb].load(g.a + oa[mb] + (uint32_t)c * 64u);
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const half8 bv = wt[slot].decode(s, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[s][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, tk[slot][mb].decode(s, 0), acc[s][mb], 0, 0, 0);
    }
  };
  // whole groups of P chunks through the ring, then the remaining chunks one
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

// Eight waves split K when it holds a multiple of eight chunks, else four.
template <class OpB, int MB>
hipError_t launch_narrow(GemmArgs& g, hipStream_t stream) {
  const long long blocks = (g.N + 31) / 32;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if ((g.K / 32) % 8 == 0)
    hipLaunchKernelGGL((narrow_kernel<OpB, MB, 8, 4>), dim3((unsigned)blocks), dim3(512), 0, stream, g);
  else
    hipLaunchKernelGGL((narrow_kernel<OpB, MB, 4, 4>), dim3((unsigned)blocks), dim3(256), 0, stream, g);
  return hipGetLastError();
}

// Narrow batches take the narrow kernel; large products the LDS-staged
// kernel (256 x 256 tiles, a ring of three 64-k chunks); the rest the
// register-fed kernel and its smaller tiles.  The staged kernel reads each
// fp16 group scale through the aligned dword that holds it, so it also needs
// a 4-byte aligned scale array with an even number of entries (else the last
// dword would reach past the array).
template <class OpB>
hipError_t launch_weight_only(GemmArgs& g, hipStream_t stream) {
  if (g.M <= 32) return launch_narrow<OpB, 1>(g, stream);
  if (g.M <= 64) return launch_narrow<OpB, 2>(g, stream);
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
