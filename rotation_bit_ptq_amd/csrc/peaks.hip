// Measured ceilings for the benchmark's roofline denominators: a loop of
// dense fp16 matrix-core products with operands held in registers (what the
// decode GEMM could at best sustain on this device, including the clock the
// matrix cores settle at under load), and the shader clock over that loop.
// Not part of the layer's C ABI: bench.py alone loads this library.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Each wave keeps kChains independent 32x32 accumulators and issues
// kChains v_mfma_f32_32x32x16_f16 per trip, so no product waits for the one
// before it.  Operands come from `seed` (random normal fp16 values give the
// matrix cores' real power draw; constant ones do not).  clocks[0..1] of
// the first wave: shader clock ticks and 100 MHz wall-clock ticks over the
// loop.
constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_loop_kernel(const uint4* seed, int trips,
                                                        float* sink, long long* clocks) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  half8 a[kChains], b[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    a[c] = __builtin_bit_cast(half8, seed[(t * 2 * kChains + 2 * c) & 4095]);
    b[c] = __builtin_bit_cast(half8, seed[(t * 2 * kChains + 2 * c + 1) & 4095]);
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[c][q] = 0.0f;
  const long long c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < trips; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[c], b[c], acc[c], 0, 0, 0);
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) s += acc[c][q];
  sink[t] = s;
  if (t == 0) {
    clocks[0] = c1 - c0;
    clocks[1] = w1 - w0;
  }
}

}  // namespace

extern "C" {

// waves_per_simd waves on every SIMD of every compute unit; returns the
// HIP status.  flops per launch = 2 * 32 * 32 * 16 * kChains * trips * waves.
int peaks_mfma_loop(const void* seed, int trips, int waves_per_simd, float* sink,
                    long long* clocks, hipStream_t stream) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (trips < 1 || waves_per_simd < 1 || waves_per_simd > 2) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_cu * waves_per_simd), dim3(256), 0, stream,
                     (const uint4*)seed, trips, sink, clocks);
  return (int)hipGetLastError();
}

int peaks_mfma_chains(void) { return kChains; }

// Rate of the wall clock read by the loop, in kHz (0 on error).
int peaks_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
