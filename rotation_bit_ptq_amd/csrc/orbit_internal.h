// Internal declarations shared by the host ABI layer and the kernel files.
#pragma once

#include <stdint.h>

#include <atomic>

#include "../../include/orbit.h"

namespace orbit {

// Per-device properties queried once (LDS per block, compute units).
struct DeviceInfo {
  int max_lds = 0;
  int n_cu = 0;
};
hipError_t device_info(DeviceInfo* out);

// One launch site's cached setup: the dynamic-LDS limit raised once per
// device, and the occupancy for the last LDS size asked about.
struct LaunchCache {
  std::atomic<unsigned long long> lds_raised{0};  // bit per device
  std::atomic<long long> occ_key{-1};             // (device << 32) | lds
  std::atomic<int> occ_blocks{0};
};
hipError_t prepare_launch(LaunchCache& c, const void* kern, int threads, int lds, int* blocks_per_cu);

// ---- rotate + quantize family (rpbh_quant.hip) ----------------------------

enum class RowMode : int {
  kActQuant = 0,     // s = ||x'||, u = sqrt(d) x' / (s + eps)
  kWeightQuant = 1,  // r = ||w'|| (bf16), u = sqrt(d) w' / r
  kRotate = 2,       // x' only
  kInt8Pack = 3,     // per-group fp16 scale, int8 codes
  kInt4Pack = 4,     // per-group fp16 scale, int4 codes (two per byte)
};

// Uniform-grid lookup that turns "count thresholds below u" into one table
// read and one compare (see rpbh_quant.hip).  Chosen on the host.
struct GridSearch {
  float a, b;   // cell = clamp(floor(fma(u, a, b)), 0, cells - 1)
  int cells;    // power of two <= kMaxGridCells
  int nthr;     // number of thresholds (levels - 1)
};
constexpr int kMaxGridCells = 2048;

struct RowJob {
  RowMode mode;
  int in_dtype;    // orbit_dtype of the rows
  int out_dtype;   // kRotate: F32 / F16
  int64_t rows;
  int d, h;
  const int32_t* perm;
  const uint32_t* sign_bits;
  const uint16_t* gather;  // the rotation's gather plan, or null
  bool perm_identity;      // the caller's promise that perm[k] == k
  const void* in;
  // quantize outputs
  int bits;
  const float* thresholds;  // host pointer (levels - 1 floats)
  GridSearch grid;
  float eps;
  uint8_t* idx_out;
  float* norm_f32_out;      // act: s
  uint16_t* norm_bf16_out;  // weight: r
  float* xrot_f32_out;      // debug / rotate F32 output
  void* rot_out;            // rotate F16 output
  // int8 outputs
  int group;
  int8_t* q_out;  // int8 codes, or int4 codes two per byte
  uint16_t* scale_out;
};

hipError_t launch_rows(const RowJob& job, hipStream_t stream);

// Gather plan of a rotation (rpbh_quant.hip): 1024 uint16 entries (64 lanes
// x 16) per round of the row, at least 4 rounds.
__host__ __device__ inline int gather_len(int d) {
  const int rounds = (d + 1023) / 1024;
  return 1024 * (rounds < 4 ? 4 : rounds);
}

// The plan's second section, after gather_len(d) entries: the matrix-core
// kernels' packed offset words (two uint16 entries per word, one word per
// pair of coordinates), for the rotations those kernels can take (h = 64 ..
// 4096; the 15-bit byte offsets need d <= 16384).
__host__ __device__ inline int mfma_words_len(int d, int h) {
  const bool hk = h == 64 || h == 128 || h == 256 || h == 512 || h == 1024 || h == 2048 || h == 4096;
  return (hk && d % 512 == 0 && d <= 16384) ? d : 0;
}
// The plan's third section, after the offset words: for the packed-code
// matrix-core kernels (h = 128 or 256 on rows of 1024 .. 16384), one uint16
// entry per input coordinate i holding the LDS byte offset of the operand
// slot that needs x[i] (the slot of permuted index k = pi^-1(i)) and, in
// bit 15, the sign flip D_k, so each lane scatters the row it loaded
// straight into operand order.
__host__ __device__ inline int scatter_len(int d, int h) {
  const bool dk = d == 1024 || d == 2048 || d == 3072 || d == 4096 || d == 8192 || d == 12288 || d == 16384;
  return ((h == 128 || (h == 256 && d % 1024 == 0)) && dk) ? d : 0;
}
hipError_t launch_gather_plan(int d, int h, const int32_t* perm, const uint32_t* sign_bits,
                              uint16_t* out, hipStream_t stream);

// ---- decode GEMMs (qgemm.hip) ----------------------------------------------

struct GemmJob {
  int kind;  // 0: codebook x codebook, 1: fp16 x int8, 2: fp16 x int4
  int64_t M, N, K;
  const uint8_t* a;        // kind 0: idx_a; kinds 1, 2: fp16 Xrot
  const uint8_t* b;        // kind 0: idx_w; kind 1: int8 q; kind 2: int4 q
  int bits_a, bits_b;      // kind 0
  const float* cent_a;     // host, 2^bits_a
  const float* cent_b;     // host, 2^bits_b
  const float* s;          // kind 0: per-row scale of A (device)
  const uint16_t* r_bf16;  // kind 0: per-row scale of B (device, bf16)
  const uint16_t* scale_f16;  // kinds 1, 2: group scales (device)
  int group;
  const void* bias;
  int bias_dtype;
  void* out;
  int out_dtype;
  int act;  // orbit_act, applied in the epilogue
};

hipError_t launch_gemm(const GemmJob& job, hipStream_t stream);

}  // namespace orbit
