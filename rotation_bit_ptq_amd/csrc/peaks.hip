// Measured ceilings for the benchmark's roofline denominators: a loop of
// dense fp16 matrix-core products with operands held in registers (what the
// decode GEMM could at best sustain on this device, including the clock the
// matrix cores settle at under load), the shader clock over that loop, and
// the LDS read throughput per compute unit for 4- and 16-byte lane reads.
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
// loop.  The ceilings use 4 chains; 8, 12 and 16 show that more
// independent work per wave does not change the rate.
constexpr int kChains = 4;

template <int kChains>
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

// LDS throughput per compute unit: 8 waves (two per SIMD) each issue
// `trips` x 8 independent reads (kind 0: 4 bytes per lane, as a decode-table
// lookup; kind 1: 16 bytes per lane, as an MFMA operand) from distinct 1 KB
// blocks, every lane in its own bank, and wait once per 8.  cycles[block]:
// shader clocks over the loop.
template <int KIND>
__global__ __launch_bounds__(512) void lds_read_kernel(int trips, unsigned* sink, long long* cycles) {
  __shared__ __align__(16) char lds[65536];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < 65536 / 4; i += 512) ((unsigned*)lds)[i] = (unsigned)i;
  __syncthreads();
  const long long c0 = clock64();
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int it = 0; it < trips; ++it) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = (it * 8 + j + w * 3) & 63;  // blocks 0..63: bytes 0 .. 65535
      if constexpr (KIND == 0) v[j].x = *(const unsigned*)(lds + blk * 1024 + lane * 4);
      else v[j] = *(const uint4*)(lds + blk * 1024 + lane * 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc.x += v[j].x;
      if constexpr (KIND == 1) {
        acc.y += v[j].y;
        acc.z += v[j].z;
        acc.w += v[j].w;
      }
    }
  }
  const long long c1 = clock64();
  sink[blockIdx.x * 512 + t] = acc.x + acc.y + acc.z + acc.w;
  if (t == 0) cycles[blockIdx.x] = c1 - c0;
}

}  // namespace

extern "C" {

// One 512-thread workgroup per compute unit running lds_read_kernel; sink
// holds n_cu * 512 uint32, cycles n_cu int64.  Bytes read per workgroup:
// 8 waves * trips * 8 * (kind 0 ? 256 : 1024).  Returns the HIP status.
int peaks_lds_read(int kind, int trips, unsigned* sink, long long* cycles, hipStream_t stream) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (trips < 1 || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
  if (kind == 0) hipLaunchKernelGGL(lds_read_kernel<0>, dim3(n_cu), dim3(512), 0, stream, trips, sink, cycles);
  else hipLaunchKernelGGL(lds_read_kernel<1>, dim3(n_cu), dim3(512), 0, stream, trips, sink, cycles);
  return (int)hipGetLastError();
}


// waves_per_simd waves on every SIMD of every compute unit; returns the
// HIP status.  flops per launch = 2 * 32 * 32 * 16 * kChains * trips * waves.
int peaks_mfma_loop(const void* seed, int trips, int waves_per_simd, float* sink,
                    long long* clocks, hipStream_t stream) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (trips < 1 || waves_per_simd < 1 || waves_per_simd > 2) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel<kChains>, dim3(n_cu * waves_per_simd), dim3(256), 0, stream,
                     (const uint4*)seed, trips, sink, clocks);
  return (int)hipGetLastError();
}

int peaks_mfma_chains(void) { return kChains; }

// The same loop with `chains` (4, 8, 12 or 16) accumulators per wave.
// flops per launch = 2 * 32 * 32 * 16 * chains * trips * waves.
int peaks_mfma_loop_chains(const void* seed, int trips, int waves_per_simd, int chains,
                           float* sink, long long* clocks, hipStream_t stream) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (trips < 1 || waves_per_simd < 1 || waves_per_simd > 2) return (int)hipErrorInvalidValue;
  const dim3 grid(n_cu * waves_per_simd), block(256);
  switch (chains) {
    case 4: hipLaunchKernelGGL(mfma_loop_kernel<4>, grid, block, 0, stream, (const uint4*)seed, trips, sink, clocks); break;
    case 8: hipLaunchKernelGGL(mfma_loop_kernel<8>, grid, block, 0, stream, (const uint4*)seed, trips, sink, clocks); break;
    case 12: hipLaunchKernelGGL(mfma_loop_kernel<12>, grid, block, 0, stream, (const uint4*)seed, trips, sink, clocks); break;
    case 16: hipLaunchKernelGGL(mfma_loop_kernel<16>, grid, block, 0, stream, (const uint4*)seed, trips, sink, clocks); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Rate of the wall clock read by the loop, in kHz (0 on error).
int peaks_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
