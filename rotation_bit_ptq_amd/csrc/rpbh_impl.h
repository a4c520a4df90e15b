// Fused RPBH rotate (+ norm split, codebook quantize, pack) over rows.
//
// OrbitQuant page, Method: x' = Pi_d x with Pi_d = blkdiag(H_h D_i) P_pi;
// s = ||x'||; the direction x'/(s + eps) is quantized by the Lloyd-Max
// codebook; weights go through the same rotation offline (W' = W Pi^T, one
// row at a time) with their norm kept in BF16.  The int8 article's packer
// (section 4: rotate, per-group scale, round) and the plain rotation reuse
// the same front end.
//
// Layout of the work (gfx950, wave64):
//   * one wave owns one row (token or weight row) at a time and loops over
//     rows with a grid stride, with the next row's HBM loads in flight while
//     the current row is transformed; no workgroup barriers on the row path;
//   * the row lands in the wave's LDS buffer twice, as x and as -x, so the
//     Rademacher sign of permuted coordinate k is part of its gather address:
//       y_k = D_k x[pi(k)] = buf[pi(k) + (D_k < 0 ? d : 0)];
//     the addresses are computed once per wave and stay in registers;
//   * bf16 rows with h = 64, 128 or 256 use a transposed gather (TrShape
//     below): every butterfly stage is a register add/sub, with one pass
//     through a per-wave LDS scratch between H_T and H_16; other shapes
//     gather 16 consecutive permuted coordinates per lane and pair lanes
//     for the stages above 16 through DPP moves or ds_swizzle;
//   * the squared norm comes from the loaded row (Pi is orthogonal) and is
//     reduced across the wave; the quantizer counts the thresholds below u
//     with one lookup in a uniform grid over u: each cell holds at most one
//     threshold, so idx = base[cell] + (t[cell] < u), the same float32
//     decision as a full count.  The cell index is read off the bits of
//     fma(u, a, b + 2^23) (a monotone rounding), clamped by v_med3;
//   * each lane writes its 16 codes as one 2*bits-byte word.
// Rows with d <= 4096 keep their gather addresses in registers (one pass
// over LDS); longer rows take long_rows_kernel, one workgroup per row.  The
// quantizing modes for bf16 rows with h = 128 and d = 1024 .. 4096 run the
// Hadamard on the matrix cores instead (rpbh_mfma.h).
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "orbit_internal.h"

namespace orbit {
namespace rows {

constexpr int kWave = 64;
constexpr int kSlot = 16;  // rotated coordinates per lane-slot
constexpr int kMaxCachedRounds = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kArgCells = 256;  // grid cells carried in the kernel arguments

struct RowArgs {
  int d, h, log2h, nslots, nrounds;
  long long rows;
  const int32_t* perm;
  const uint32_t* sign_bits;
  const uint16_t* gather;  // gather plan in this kernel's order, or null
  const uint32_t* mfma_words;  // the plan's matrix-core offset words, or null
  const uint32_t* scatter_words;  // the plan's scatter section (two entries per word), or null
  int perm_identity;       // 1: perm[k] == k (the matrix-core kernels read rows directly)
  const void* in;
  float sqrt_d_over_h;  // sqrt(d / h): u = z * sqrt(d/h) / (s + eps), z = H y unnormalised
  float sqrt_h_over_d;  // its reciprocal: 1 / alpha = (s + eps) * sqrt(h/d)
  float inv_sqrt_h;
  float inv_h;
  float eps;
  float ga, gb;  // gb already includes 2^23
  int cells, nthr;
  uint32_t grid_bias;  // 0xA8000000: turns the cell's float bits into its byte offset
  int cells_in_args;   // 1: the grid table below was built on the host
  float thr[ORBIT_MAX_LEVELS - 1];
  uint8_t* idx_out;
  float* s_out;
  uint16_t* r_out;
  float* xrot_f32;
  uint16_t* xrot_f16;
  int group;
  int8_t* q_out;
  uint16_t* scale_out;
  int grid_bytes;   // LDS bytes of the grid table
  int row_bytes;    // LDS bytes of one wave's row buffer (x and -x)
  int wave_bytes;   // row buffer + transpose scratch of one wave
  float cell_t[kArgCells];       // host-built grid (cells_in_args): thresholds
  uint8_t cell_base[kArgCells];  // and counts of thresholds in lower cells
};
static_assert(sizeof(RowArgs) <= 4096, "kernel arguments must stay within 4 KB");

enum Mode { kAct = 0, kWeight = 1, kRotF32 = 2, kRotF16 = 3, kInt8 = 4, kInt4 = 5 };

struct GridCell {
  float t;   // the threshold inside the cell, +inf if none
  int base;  // thresholds in lower cells
};


constexpr float kMagic = 8388608.0f;  // 2^23: floats in [2^23, 2^24) are integers

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// The grid cell of u: the float fma(u, a, b + 2^23) rounded to an integer,
// clamped to [2^23, 2^23 + cells - 1]; returns the cell's LDS byte address
// (the grid table starts at LDS byte 0, 8 bytes per cell):
// (bits - 0x4B000000) * 8 = bits * 8 + bias, bias = 0xA8000000 (mod 2^32),
// passed in as a kernel argument so it sits in a scalar register.
__device__ __forceinline__ uint32_t grid_addr(float u, float a, float b, float top, uint32_t bias) {
  float f = __builtin_fmaf(u, a, b);
  f = __builtin_amdgcn_fmed3f(f, kMagic, top);
  return (__float_as_uint(f) << 3) + bias;
}

__device__ __forceinline__ int grid_index(float u, float a, float b, float top) {
  float f = __builtin_amdgcn_fmed3f(__builtin_fmaf(u, a, b), kMagic, top);
  return (int)(__float_as_uint(f) - 0x4B000000u);
}

// Sum over the wave, identical in every lane and independent of timing:
// DPP butterflies inside each row of 16 lanes, then the four row sums are
// read as scalars and added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // xor 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // xor 2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float group_max(float v, int lanes) {
  for (int m = 1; m < lanes; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Orders a wave's LDS writes before its later reads (a wave's LDS
// operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of lane ^ M.
template <int M>
__device__ __forceinline__ float xor_partner(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  if constexpr (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x101F));
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));
  if constexpr (M == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));
  if constexpr (M == 32) return __shfl_xor(v, 32, kWave);
  return v;
}

// Butterfly between lanes j and j ^ M: the lower lane keeps a + b, the
// upper one a - b (its partner holds a).  Written as partner + v * sign with
// contraction off, so the DPP move folds into the add's source operand and
// the add's result may land in any register.
template <int M>
__device__ __forceinline__ void lane_stage(float (&v)[kSlot], int lane) {
#pragma clang fp contract(off)
  const float sg = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < kSlot; ++i) {
    const float t = v[i] * sg;
    v[i] = xor_partner<M>(v[i]) + t;
  }
}

__device__ __forceinline__ void lane_stages(float (&v)[kSlot], int lane, int nstages) {
  if (nstages > 0) lane_stage<1>(v, lane);
  if (nstages > 1) lane_stage<2>(v, lane);
  if (nstages > 2) lane_stage<4>(v, lane);
  if (nstages > 3) lane_stage<8>(v, lane);
  if (nstages > 4) lane_stage<16>(v, lane);
  if (nstages > 5) lane_stage<32>(v, lane);
}

// Blocks longer than one round (h = 1024 n, n = 2 or 4): in Sylvester order
// H_h = H_n (x) H_1024 and round r holds positions 1024 r .. 1024 r + 1023,
// so after H_1024 inside every round the remaining stages pair rounds
// r and r + span, element by element, in registers.
template <int R>
__device__ __forceinline__ void round_stages(float (&v)[R][kSlot], int n) {
#pragma unroll
  for (int span = 1; span < R; span <<= 1) {
    if (span >= n) break;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r & span) continue;
#pragma unroll
      for (int i = 0; i < kSlot; ++i) {
        const float x = v[r][i], y = v[r + span][i];
        v[r][i] = x + y;
        v[r + span][i] = x - y;
      }
    }
  }
}

// Butterfly stages of span `from` .. 8 inside the lane's 16 values.
__device__ __forceinline__ void slot_stages(float (&v)[kSlot], int from) {
#pragma unroll
  for (int span = 1; span < kSlot; span <<= 1) {
    if (span < from) continue;
#pragma unroll
    for (int i = 0; i < kSlot; ++i) {
      if ((i & span) == 0) {
        float x = v[i], y = v[i + span];
        v[i] = x + y;
        v[i + span] = x - y;
      }
    }
  }
}

template <typename InT>
__device__ __forceinline__ float lds_value(const char* smem, uint32_t addr) {
  if constexpr (sizeof(InT) == 2) return __uint_as_float((uint32_t)(*(const uint16_t*)(smem + addr)) << 16);
  else return *(const float*)(smem + addr);
}

// Gathers the lane's 16 permuted, signed coordinates and applies H_16.
template <typename InT>
__device__ __forceinline__ void gather_h16(const char* smem, const uint32_t (&addr)[kSlot],
                                           float (&v)[kSlot]) {
#pragma unroll
  for (int i = 0; i < kSlot; ++i) v[i] = lds_value<InT>(smem, addr[i]);
  slot_stages(v, 1);
}

// LDS byte addresses of y_k = D_k x[pi(k)] for k = 16 slot .. 16 slot + 15.
template <typename InT>
__device__ __forceinline__ void slot_addresses(const RowArgs& a, int slot, uint32_t wbuf,
                                               uint32_t (&addr)[kSlot]) {
  const int k0 = (slot < a.nslots ? slot : 0) * kSlot;
  const i32x4* pp = (const i32x4*)(a.perm + k0);
  const i32x4 p0 = pp[0], p1 = pp[1], p2 = pp[2], p3 = pp[3];
  const uint32_t sw = a.sign_bits[k0 >> 5] >> (k0 & 31);  // 16 signs (k0 % 16 == 0)
  const int p[kSlot] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w,
                        p2.x, p2.y, p2.z, p2.w, p3.x, p3.y, p3.z, p3.w};
#pragma unroll
  for (int i = 0; i < kSlot; ++i)
    addr[i] = wbuf + ((uint32_t)p[i] + ((sw >> i) & 1u) * (uint32_t)a.d) * (uint32_t)sizeof(InT);
}

// ---- transposed gather (h = 16 T, T = 2^LT lanes per Hadamard block) ----
// Position p of a block is split as p = 16 t + i (t < T, i < 16); since
// H_h = H_T (x) H_16 in Sylvester order, the transform is H_T over t for
// every i, then H_16 over i for every t.  Lane t' of the block's T lanes
// first gathers p = 16 t + G t' + i' (all t, i' < G = 16 / T) and runs H_T
// in registers; one pass through a per-wave LDS scratch then hands every
// lane its 16 consecutive positions 16 t' .. 16 t' + 15 for H_16, again in
// registers.  Every butterfly stage is a register add/sub.
template <int LT>
struct TrShape {
  static constexpr int T = 1 << LT;       // lanes per block
  static constexpr int G = 16 >> LT;      // i values per lane before the transpose
  static constexpr int LG = 4 - LT;       // element bits that index i'
  static constexpr int P = 20;            // scratch words per lane (16 + 4 padding)
  static constexpr int S = P * T + 4;     // scratch words per block
  static constexpr int kScratchBytes = (kWave / T) * S * 4;
};

// Permuted index k of element e = t G + i' of the lane's gather.
template <int LT>
__device__ __forceinline__ int tr_k(int slot, int e) {
  using Sh = TrShape<LT>;
  const int tp = slot & (Sh::T - 1);
  return (slot - tp) * kSlot + kSlot * (e >> Sh::LG) + Sh::G * tp + (e & (Sh::G - 1));
}

template <typename InT, int LT>
__device__ __forceinline__ void tr_addresses(const RowArgs& a, int slot, uint32_t wbuf,
                                             uint32_t (&addr)[kSlot]) {
  const int s = slot < a.nslots ? slot : 0;
#pragma unroll
  for (int e = 0; e < kSlot; ++e) {
    const int k = tr_k<LT>(s, e);
    const uint32_t p = (uint32_t)a.perm[k];
    const uint32_t neg = (a.sign_bits[k >> 5] >> (k & 31)) & 1u;
    addr[e] = wbuf + (p + neg * (uint32_t)a.d) * (uint32_t)sizeof(InT);
  }
}

// Butterflies over element-index bits [lo, 4) (bit b pairs e and e ^ 2^b).
template <int LO>
__device__ __forceinline__ void elem_stages(float (&v)[kSlot]) {
#pragma unroll
  for (int span = 1 << LO; span < kSlot; span <<= 1) {
#pragma unroll
    for (int e = 0; e < kSlot; ++e) {
      if ((e & span) == 0) {
        float x = v[e], y = v[e + span];
        v[e] = x + y;
        v[e + span] = x - y;
      }
    }
  }
}

// Gather, H_T, transpose, H_16: v ends as the lane's 16 consecutive
// positions of x' (unnormalised).  `scr` is the wave scratch's byte offset.
template <typename InT, int LT>
__device__ __forceinline__ void tr_rotate(char* smem, uint32_t scr, const uint32_t (&addr)[kSlot],
                                          float (&v)[kSlot], int lane) {
  using Sh = TrShape<LT>;
#pragma unroll
  for (int e = 0; e < kSlot; ++e) v[e] = lds_value<InT>(smem, addr[e]);
  elem_stages<Sh::LG>(v);  // H_T over t = e >> LG
  const int tp = lane & (Sh::T - 1);
  const uint32_t grp = scr + (uint32_t)((lane >> LT) * Sh::S) * 4u;
  // writer layout: word P tp + e of the block's scratch.  A padded lane
  // stride of 20 words puts the lanes of a block on distinct bank quads and
  // the block stride S shifts blocks against each other.  The reads below
  // follow the writes in program order; a wave's LDS operations complete in
  // order and the two address sets may alias, so they are not reordered.
  float4* w = (float4*)(smem + grp + 4u * Sh::P * (uint32_t)tp);
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  // position 16 tp + G tq + i' sits in writer tq's element tp G + i'
  const char* rd = smem + grp + 4u * (uint32_t)(Sh::G * tp);
#pragma unroll
  for (int tq = 0; tq < Sh::T; ++tq) {
    const float* src = (const float*)(rd + 4 * Sh::P * tq);
    if constexpr (Sh::G == 4) {
      float4 q = *(const float4*)src;
      v[4 * tq] = q.x; v[4 * tq + 1] = q.y; v[4 * tq + 2] = q.z; v[4 * tq + 3] = q.w;
    } else if constexpr (Sh::G == 2) {
      float2 q = *(const float2*)src;
      v[2 * tq] = q.x; v[2 * tq + 1] = q.y;
    } else {
      v[tq] = src[0];
    }
  }
  elem_stages<0>(v);       // H_16 over i
}

template <int BITS>
__device__ __forceinline__ void store_indices(uint8_t* row_out, int slot, const int (&idx)[kSlot]) {
  constexpr int kWords = (kSlot * BITS + 31) / 32;
  uint32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) w[i] = 0;
#pragma unroll
  for (int i = 0; i < kSlot; ++i) {
    const int bit = i * BITS;
    w[bit / 32] |= (uint32_t)idx[i] << (bit % 32);
    if ((bit % 32) + BITS > 32) w[bit / 32 + 1] |= (uint32_t)idx[i] >> (32 - bit % 32);
  }
  uint8_t* p = row_out + (size_t)slot * (2 * BITS);
  if constexpr (BITS == 8) {
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (BITS == 4) {
    *(uint2*)p = make_uint2(w[0], w[1]);
  } else if constexpr (BITS == 2) {
    *(uint32_t*)p = w[0];
  } else if constexpr (BITS == 6) {
    uint32_t* q = (uint32_t*)p;  // 12-byte words, 4-byte aligned
    q[0] = w[0];
    q[1] = w[1];
    q[2] = w[2];
  } else if constexpr (BITS == 3) {
    uint16_t* q = (uint16_t*)p;  // 6-byte words, 2-byte aligned
    q[0] = (uint16_t)w[0];
    q[1] = (uint16_t)(w[0] >> 16);
    q[2] = (uint16_t)w[1];
  } else {
    static_assert(BITS == 1, "unsupported width");
    *(uint16_t*)p = (uint16_t)w[0];
  }
}

// A row in flight: the lane's 16-byte chunks c = lane + 64 j.
template <typename InT, int NCH>
struct RowRegs {
  u32x4 c[NCH];

  __device__ __forceinline__ void load(const RowArgs& a, long long row, int lane) {
    const int nchunk = a.d * (int)sizeof(InT) / 16;
    const u32x4* src = (const u32x4*)((const char*)a.in + (size_t)row * a.d * sizeof(InT));
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = lane + kWave * j;
      c[j] = __builtin_nontemporal_load(src + (ch < nchunk ? ch : 0));
    }
  }

  // Sum of squares of the lane's coordinates.  Pi is orthogonal, so the
  // row's sum over the wave is ||x'||^2 = ||x||^2 and the norm is known
  // before the rotation.  bf16 pairs go through v_dot2c_f32_bf16 (exact
  // products, one rounding per pair); chunks past the row end count zero.
  __device__ __forceinline__ float sumsq(const RowArgs& a, int lane) const {
    const int nchunk = a.d * (int)sizeof(InT) / 16;
    float ss = 0.0f;
    if (nchunk == NCH * kWave) {  // uniform: every chunk is part of the row
#pragma unroll
      for (int j = 0; j < NCH; ++j) ss = chunk_sumsq(c[j], ss);
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        if (lane + kWave * j < nchunk) ss = chunk_sumsq(c[j], ss);
    }
    return ss;
  }

  static __device__ __forceinline__ float chunk_sumsq(const u32x4& v, float ss) {
    // the dwords go through a scalar array: a bit_cast of a subscripted
    // vector element (v[q]) is compiled as v[0] for every q here
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (sizeof(InT) == 2) {
        const bf16x2 p = __builtin_bit_cast(bf16x2, w[q]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
      } else {
        const float f = __uint_as_float(w[q]);
        ss = __builtin_fmaf(f, f, ss);
      }
    }
    return ss;
  }

  // writes x and -x into the wave's buffer
  __device__ __forceinline__ void store(const RowArgs& a, char* smem, uint32_t wbuf, int lane) const {
    const int nchunk = a.d * (int)sizeof(InT) / 16;
    const uint32_t negoff = (uint32_t)a.d * (uint32_t)sizeof(InT);
    const uint32_t flip = sizeof(InT) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = lane + kWave * j;
      if (ch < nchunk) {
        *(u32x4*)(smem + wbuf + ch * 16) = c[j];
        *(u32x4*)(smem + wbuf + negoff + ch * 16) = c[j] ^ flip;
      }
    }
  }
};

// kXrot: also write the debug copy of x' (activation mode); chosen by a
// uniform branch around the whole row so that the plain path carries none of
// its arithmetic.
template <int MODE, int BITS, bool kXrot = false>
__device__ __forceinline__ void emit_slot(const RowArgs& a, long long row, int slot, int lane,
                                          float (&v)[kSlot], float alpha, const char* smem) {
  const int d = a.d;
  if constexpr (MODE == kAct || MODE == kWeight) {
    const float top = kMagic + (float)(a.cells - 1);
    int idx[kSlot];
#pragma unroll
    for (int i = 0; i < kSlot; ++i) {
      const float u = v[i] * alpha;
      const GridCell g = *(const GridCell*)(smem + grid_addr(u, a.ga, a.gb, top, a.grid_bias));
      idx[i] = g.base + (g.t < u ? 1 : 0);
    }
    store_indices<BITS>(a.idx_out + (size_t)row * ((size_t)d * BITS / 8), slot, idx);
    if constexpr (MODE == kAct && kXrot) {
      float4* o = (float4*)(a.xrot_f32 + (size_t)row * d + slot * kSlot);
#pragma unroll
      for (int i = 0; i < kSlot; i += 4)
        o[i / 4] = make_float4(v[i] * a.inv_sqrt_h, v[i + 1] * a.inv_sqrt_h,
                               v[i + 2] * a.inv_sqrt_h, v[i + 3] * a.inv_sqrt_h);
    }
  } else if constexpr (MODE == kRotF32) {
    float4* o = (float4*)(a.xrot_f32 + (size_t)row * d + slot * kSlot);
#pragma unroll
    for (int i = 0; i < kSlot; i += 4)
      o[i / 4] = make_float4(v[i] * a.inv_sqrt_h, v[i + 1] * a.inv_sqrt_h,
                             v[i + 2] * a.inv_sqrt_h, v[i + 3] * a.inv_sqrt_h);
  } else if constexpr (MODE == kRotF16) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (uint32_t)f32_to_f16_rne(v[2 * i] * a.inv_sqrt_h) |
             ((uint32_t)f32_to_f16_rne(v[2 * i + 1] * a.inv_sqrt_h) << 16);
    uint4* o = (uint4*)(a.xrot_f16 + (size_t)row * d + slot * kSlot);
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {  // kInt8 / kInt4: per-group symmetric scale, round half to even
    static_assert(MODE == kInt8 || MODE == kInt4, "unknown mode");
    constexpr float kQmax = MODE == kInt8 ? 127.0f : 7.0f;
    constexpr int kCodeBits = MODE == kInt8 ? 8 : 4;  // two's complement
    float w[kSlot];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kSlot; ++i) {
      w[i] = v[i] * a.inv_sqrt_h;
      amax = fmaxf(amax, fabsf(w[i]));
    }
    const int lanes = a.group / kSlot;  // lanes per group, a power of two <= 64
    amax = group_max(amax, lanes);
    const uint16_t sbits = f32_to_f16_rne(amax / kQmax);
    const float sc = (float)__builtin_bit_cast(_Float16, sbits);
    uint32_t q4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kSlot; ++i) {
      float qf = 0.0f;
      if (sc > 0.0f) qf = fminf(fmaxf(__builtin_rintf(w[i] / sc), -kQmax), kQmax);
      constexpr int kPer = 32 / kCodeBits;
      q4[i / kPer] |= ((uint32_t)(int)qf & ((1u << kCodeBits) - 1u)) << (kCodeBits * (i % kPer));
    }
    uint8_t* q_row = (uint8_t*)a.q_out + (size_t)row * ((size_t)d * kCodeBits / 8);
    if constexpr (MODE == kInt8) *(uint4*)(q_row + slot * kSlot) = make_uint4(q4[0], q4[1], q4[2], q4[3]);
    else *(uint2*)(q_row + slot * (kSlot / 2)) = make_uint2(q4[0], q4[1]);
    if ((lane & (lanes - 1)) == 0)
      a.scale_out[(size_t)row * (d / a.group) + slot * kSlot / a.group] = sbits;
  }
}

// ss: the sum of squares of x (kFromInput) or of the unnormalised rotated
// values z = sqrt(h) x' (one pass per row of the long-row path).
template <int MODE, bool kFromInput = false>
__device__ __forceinline__ float row_alpha(const RowArgs& a, float ss, long long row, int lane) {
  if constexpr (!kFromInput) ss *= a.inv_h;
  if constexpr (MODE == kAct) {
    float s = sqrtf(ss);
    if (lane == 0) a.s_out[row] = s;
    return a.sqrt_d_over_h / (s + a.eps);
  } else if constexpr (MODE == kWeight) {
    float r = sqrtf(ss);
    if (lane == 0) a.r_out[row] = f32_to_bf16_rne(r);
    return r > 0.0f ? a.sqrt_d_over_h / r : 0.0f;
  } else {
    return 0.0f;
  }
}

// As row_alpha, and 1 / alpha for the per-row threshold rewrite: for
// activations (s + eps) sqrt(h/d), one multiply instead of a division on
// the row's dependency chain (both round within a few float32 ulps of the
// exact quotient); for weights 1 / alpha as before (a zero row gives an
// infinite factor, so its thresholds keep their signs).
template <int MODE>
__device__ __forceinline__ float row_alpha_inv(const RowArgs& a, float ss, long long row, int lane,
                                               float& inv) {
  if constexpr (MODE == kAct) {
    const float s = sqrtf(ss);
    if (lane == 0) a.s_out[row] = s;
    const float se = s + a.eps;
    inv = se * a.sqrt_h_over_d;
    return a.sqrt_d_over_h / se;
  } else {
    const float alpha = row_alpha<MODE, true>(a, ss, row, lane);
    inv = 1.0f / alpha;
    return alpha;
  }
}

// Grid table: cell c holds the unique threshold the float32 classification
// puts in it (if any) and the number of thresholds in lower cells.  Grids of
// up to kArgCells cells are built on the host with the same float32 cell
// function and copied from the kernel arguments; larger ones are built here,
// reading the thresholds in a uniform loop (scalar loads), never with
// per-lane indices.
__device__ __forceinline__ void build_grid(const RowArgs& a, char* smem) {
  if (a.cells_in_args) {
    for (int c = threadIdx.x; c < a.cells; c += blockDim.x) {
      GridCell g;
      g.t = a.cell_t[c];
      g.base = a.cell_base[c];
      ((GridCell*)smem)[c] = g;
    }
    return;
  }
  const float top = kMagic + (float)(a.cells - 1);
  for (int c = threadIdx.x; c < a.cells; c += blockDim.x) {
    GridCell g;
    g.base = 0;
    g.t = INFINITY;
    for (int j = 0; j < a.nthr; ++j) {
      const float t = a.thr[j];
      const int cj = grid_index(t, a.ga, a.gb, top);
      g.base += (cj < c) ? 1 : 0;
      if (cj == c) g.t = t;
    }
    ((GridCell*)smem)[c] = g;
  }
}

// Position of coordinate k in the workgroup's offset table: one pad word per
// 128 entries, so the lane groups of a wave (whose indices differ by
// multiples of 128) read different banks.
__device__ __forceinline__ int off_slot(int k) { return k + (k >> 7); }

// Byte offsets of the signed, permuted coordinates in a wave's row buffer,
// computed once per workgroup: off[k] = (pi(k) + (D_k < 0 ? d : 0)) * size,
// so y_k = D_k x[pi(k)] sits at wbuf + off[k].  One coalesced pass over
// pi and the sign bits instead of per-lane scattered loads in every wave.
template <typename InT>
__device__ __forceinline__ void block_offsets(const RowArgs& a, uint32_t* off) {
  for (int k = threadIdx.x; k < a.d; k += blockDim.x) {
    const uint32_t neg = (a.sign_bits[k >> 5] >> (k & 31)) & 1u;
    off[off_slot(k)] = ((uint32_t)a.perm[k] + neg * (uint32_t)a.d) * (uint32_t)sizeof(InT);
  }
}

// The lane's gather addresses of one round from the workgroup's offsets.
template <typename InT, int LT>
__device__ __forceinline__ void lds_addresses(const RowArgs& a, const uint32_t* off, int slot,
                                              uint32_t wbuf, uint32_t (&addr)[kSlot]) {
  const int s = slot < a.nslots ? slot : 0;
  if constexpr (LT >= 0) {
#pragma unroll
    for (int e = 0; e < kSlot; ++e) addr[e] = wbuf + off[off_slot(tr_k<LT>(s, e))];
  } else {
#pragma unroll
    for (int e = 0; e < kSlot; ++e) addr[e] = wbuf + off[off_slot(s * kSlot + e)];
  }
}

// R > 0: rows of at most 1024 R coordinates, values and addresses in
// registers.  R == 0: longer rows, two passes over the LDS copy.
// LT >= 0: transposed gather with T = 2^LT lanes per Hadamard block (h =
// 16 T); LT < 0: consecutive gather with cross-lane butterfly stages.
template <typename InT, int MODE, int BITS, int R, int LT>
__global__ __launch_bounds__(256) void rows_kernel(RowArgs a) {
  static_assert(R > 0, "rows longer than 4096 coordinates take long_rows_kernel");
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t wbuf = (uint32_t)(a.grid_bytes + wave * a.wave_bytes);
  const uint32_t scr = wbuf + (uint32_t)a.row_bytes;  // transpose scratch (LT >= 0)
  const long long stride = (long long)gridDim.x * waves;
  long long row = (long long)blockIdx.x * waves + wave;
  const int nstages = a.log2h - 4;
  constexpr bool kQuant = (MODE == kAct || MODE == kWeight);

  if constexpr (R > 0) {
    constexpr int NCH = R * (int)sizeof(InT);  // 16-byte chunks per lane
    RowRegs<InT, NCH> pre;
    uint32_t addr[R][kSlot];
    if (a.gather) {  // uniform: the rotation's gather plan, 32 bytes per lane and round
      u32x4 gp[R][2];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const u32x4* src = (const u32x4*)(a.gather + r * 1024 + lane * kSlot);
        gp[r][0] = src[0];
        gp[r][1] = src[1];
      }
      if (row < a.rows) pre.load(a, row, lane);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w[8] = {gp[r][0].x, gp[r][0].y, gp[r][0].z, gp[r][0].w,
                               gp[r][1].x, gp[r][1].y, gp[r][1].z, gp[r][1].w};
#pragma unroll
        for (int e = 0; e < kSlot; ++e)
          addr[r][e] = wbuf + ((w[e >> 1] >> (16 * (e & 1))) & 0xffffu) * (uint32_t)sizeof(InT);
      }
      if constexpr (kQuant) {
        build_grid(a, smem);
        __syncthreads();
      }
    } else {
    // Gather offsets (overlaying the row buffers until the first row lands)
    // and the grid table, then every lane's addresses.  The loads of pi and
    // the sign bits are issued before the first row's, so waiting for them
    // does not wait for the row.
    // 256 threads: thread t owns coordinates 4 t + 1024 i .. + 3 (i < R), read
    // as one 16-byte load of pi each, and the sign word of each group.
    const bool full = blockDim.x == 256;  // uniform
    i32x4 pv[R];
    uint32_t sv[R];
    if (full) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int k0 = 4 * (int)threadIdx.x + 1024 * i;
        pv[i] = k0 < a.d ? *(const i32x4*)(a.perm + k0) : i32x4{0, 0, 0, 0};
        sv[i] = k0 < a.d ? a.sign_bits[k0 >> 5] : 0u;
      }
    }
    if (row < a.rows) pre.load(a, row, lane);
    uint32_t* const off = (uint32_t*)(smem + a.grid_bytes);
    if (full) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int k0 = 4 * (int)threadIdx.x + 1024 * i;
        if (k0 < a.d) {
          const int pk[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k = k0 + q;
            off[off_slot(k)] = ((uint32_t)pk[q] + ((sv[i] >> (k & 31)) & 1u) * (uint32_t)a.d) * (uint32_t)sizeof(InT);
          }
        }
      }
    } else {
      block_offsets<InT>(a, off);
    }
    if constexpr (kQuant) build_grid(a, smem);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) lds_addresses<InT, LT>(a, off, r * kWave + lane, wbuf, addr[r]);
    __syncthreads();
    }
    for (; row < a.rows; row += stride) {
      float ssx = 0.0f;
      if constexpr (kQuant) ssx = pre.sumsq(a, lane);
      pre.store(a, smem, wbuf, lane);
      if (row + stride < a.rows) pre.load(a, row + stride, lane);
      // the norm first: its wave reduction overlaps the rotation below
      float alpha = 0.0f;
      if constexpr (kQuant) alpha = row_alpha<MODE, true>(a, wave_sum(ssx), row, lane);
      wave_lds_sync();
      float v[R][kSlot];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (LT >= 0) {
          tr_rotate<InT, LT>(smem, scr, addr[r], v[r], lane);
        } else {
          gather_h16<InT>(smem, addr[r], v[r]);
          lane_stages(v[r], lane, nstages);
        }
      }
      if constexpr (LT < 0 && R > 1) {
        if (a.h > 1024) round_stages<R>(v, a.h >> 10);  // uniform: h = 2048, 4096
      }
      wave_lds_sync();  // every lane has gathered before the next row lands
      // uniform branches: the debug copy of x', and whether every lane of
      // every round holds a slot of the row
      auto emit_all = [&](auto xrot) {
        constexpr bool kX = decltype(xrot)::value;
        if (a.nslots == R * kWave) {
#pragma unroll
          for (int r = 0; r < R; ++r) emit_slot<MODE, BITS, kX>(a, row, r * kWave + lane, lane, v[r], alpha, smem);
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int slot = r * kWave + lane;
            if (slot < a.nslots) emit_slot<MODE, BITS, kX>(a, row, slot, lane, v[r], alpha, smem);
          }
        }
      };
      if (MODE == kAct && a.xrot_f32) emit_all(std::true_type{});
      else emit_all(std::false_type{});
    }
  }
}

// Rows longer than 4096 coordinates: one workgroup of four waves per row.
// The row lands once in a shared LDS buffer (as x and -x), its norm comes
// from the loaded values through a fixed-order workgroup reduction, and the
// rounds of 1024 coordinates are split across the waves; the next row's
// loads are in flight meanwhile.  One pass over the row.
template <typename InT, int MODE, int BITS, int LT>
__global__ __launch_bounds__(256) void long_rows_kernel(RowArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr bool kQuant = (MODE == kAct || MODE == kWeight);
  constexpr int kPer = ORBIT_MAX_D * (int)sizeof(InT) / 16 / 256;  // 16-byte chunks per thread
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  float* const red = (float*)(smem + a.grid_bytes);         // four wave sums
  const uint32_t rbuf = (uint32_t)a.grid_bytes + 16u;        // the row, x then -x
  uint32_t scr = 0;
  if constexpr (LT >= 0) scr = rbuf + (uint32_t)a.row_bytes + (uint32_t)(wave * TrShape<LT>::kScratchBytes);
  const int nchunk = a.d * (int)sizeof(InT) / 16;
  const uint32_t negoff = (uint32_t)a.d * (uint32_t)sizeof(InT);
  const uint32_t flip = sizeof(InT) == 2 ? 0x80008000u : 0x80000000u;
  const int nstages = a.log2h - 4;
  if constexpr (kQuant) build_grid(a, smem);  // visible after the first barrier below

  u32x4 pre[kPer];
  auto load = [&](long long rr) {
    const u32x4* src = (const u32x4*)((const char*)a.in + (size_t)rr * a.d * sizeof(InT));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = t + 256 * i;
      if (ch < nchunk) pre[i] = __builtin_nontemporal_load(src + ch);
    }
  };
  long long row = blockIdx.x;
  if (row < a.rows) load(row);
  for (; row < a.rows; row += gridDim.x) {
    float ssx = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = t + 256 * i;
      if (ch < nchunk) {
        if constexpr (kQuant) ssx = RowRegs<InT, 1>::chunk_sumsq(pre[i], ssx);
        *(u32x4*)(smem + rbuf + ch * 16) = pre[i];
        *(u32x4*)(smem + rbuf + negoff + ch * 16) = pre[i] ^ flip;
      }
    }
    if (row + gridDim.x < a.rows) load(row + gridDim.x);
    if constexpr (kQuant) {
      const float ws = wave_sum(ssx);
      if (lane == 0) red[wave] = ws;
    }
    __syncthreads();  // the row and the wave sums are in LDS
    float alpha = 0.0f;
    if constexpr (kQuant) alpha = row_alpha<MODE, true>(a, (red[0] + red[1]) + (red[2] + red[3]), row, t);
    for (int r = wave; r < a.nrounds; r += 4) {
      const int slot = r * kWave + lane;
      uint32_t addr[kSlot];
      float v[kSlot];
      if (a.gather) {  // uniform
        const u32x4* src = (const u32x4*)(a.gather + r * 1024 + lane * kSlot);
        const u32x4 g0 = src[0], g1 = src[1];
        const uint32_t w[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int e = 0; e < kSlot; ++e)
          addr[e] = rbuf + ((w[e >> 1] >> (16 * (e & 1))) & 0xffffu) * (uint32_t)sizeof(InT);
      } else if constexpr (LT >= 0) {
        tr_addresses<InT, LT>(a, slot, rbuf, addr);
      } else {
        slot_addresses<InT>(a, slot, rbuf, addr);
      }
      if constexpr (LT >= 0) {
        tr_rotate<InT, LT>(smem, scr, addr, v, lane);
      } else {
        gather_h16<InT>(smem, addr, v);
        lane_stages(v, lane, nstages);
      }
      if (slot < a.nslots) {
        if (MODE == kAct && a.xrot_f32) emit_slot<MODE, BITS, true>(a, row, slot, lane, v, alpha, smem);
        else emit_slot<MODE, BITS>(a, row, slot, lane, v, alpha, smem);
      }
    }
    __syncthreads();  // every wave has gathered before the next row lands
  }
}

template <typename InT, int MODE, int BITS, int LT>
hipError_t launch_long(RowArgs a, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  if (a.d > ORBIT_MAX_D) return hipErrorInvalidValue;
  int lds = a.grid_bytes + 16 + a.row_bytes;
  if constexpr (LT >= 0) lds += 4 * TrShape<LT>::kScratchBytes;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  auto kern = long_rows_kernel<InT, MODE, BITS, LT>;
  static LaunchCache cache;
  int per_cu = 1;
  e = prepare_launch(cache, (const void*)kern, 256, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <typename InT, int MODE, int BITS, int R, int LT>
hipError_t launch_typed(RowArgs a, hipStream_t stream) {
  if constexpr (R == 0) {
    return launch_long<InT, MODE, BITS, LT>(a, stream);
  } else {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  if constexpr (LT >= 0) a.wave_bytes = a.row_bytes + TrShape<LT>::kScratchBytes;
  else a.wave_bytes = a.row_bytes;
  int waves = 4;
  while (waves > 1 && a.grid_bytes + waves * a.wave_bytes > di.max_lds) waves >>= 1;
  const int lds = a.grid_bytes + waves * a.wave_bytes;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  // the gather offsets (4 bytes per coordinate plus a pad word per 128)
  // overlay the row buffers
  if (R > 0 && 4LL * (a.d + a.d / 128 + 1) > (long long)waves * a.wave_bytes) return hipErrorInvalidValue;
  auto kern = rows_kernel<InT, MODE, BITS, R, LT>;
  static LaunchCache cache;
  int per_cu = 1;
  e = prepare_launch(cache, (const void*)kern, waves * kWave, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long need = (a.rows + waves - 1) / waves;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(need < cap ? need : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(waves * kWave), lds, stream, a);
  return hipGetLastError();
  }
}

// Register-resident rounds for a row of d coordinates (0 = the long-row
// kernel, one workgroup per row).
inline int rounds_for(int d) {
  const int r = (d / kSlot + kWave - 1) / kWave;
  return r <= kMaxCachedRounds ? r : 0;
}

template <typename InT, int MODE, int BITS>
hipError_t launch_rounds(const RowArgs& a, hipStream_t stream) {
  switch (rounds_for(a.d)) {
    case 1: return launch_typed<InT, MODE, BITS, 1, -1>(a, stream);
    case 2: return launch_typed<InT, MODE, BITS, 2, -1>(a, stream);
    case 3: return launch_typed<InT, MODE, BITS, 3, -1>(a, stream);
    case 4: return launch_typed<InT, MODE, BITS, 4, -1>(a, stream);
    default: return launch_typed<InT, MODE, BITS, 0, -1>(a, stream);
  }
}

// Transposed-gather kernels for bf16 rows, h = 16 * 2^LT; rows of up to
// 2048 coordinates share the two-round instantiation.
template <int MODE, int BITS, int LT>
hipError_t launch_fast_rounds(const RowArgs& a, hipStream_t stream) {
  const int r = rounds_for(a.d);
  if (r == 1 || r == 2) return launch_typed<uint16_t, MODE, BITS, 2, LT>(a, stream);
  if (r == 3) return launch_typed<uint16_t, MODE, BITS, 3, LT>(a, stream);
  if (r == 4) return launch_typed<uint16_t, MODE, BITS, 4, LT>(a, stream);
  return launch_typed<uint16_t, MODE, BITS, 0, LT>(a, stream);
}

template <int MODE, int LT>
hipError_t launch_fast(const RowArgs& a, int bits, hipStream_t stream);

// Matrix-core kernels (rpbh_mfma.h): bf16 rows, h = 32 G (64, 128, 256),
// d = 1024, 2048, 3072 or 4096, codebook modes, code widths 2, 3, 4, 6, 8.
template <int MODE, int G>
hipError_t launch_mfma(const RowArgs& a, int bits, hipStream_t stream);

#define ORBIT_ROWS_FAST(MODE, LT)                                             \
  template <>                                                               \
  hipError_t launch_fast<MODE, LT>(const RowArgs& a, int bits, hipStream_t s) { \
    switch (bits) {                                                         \
      case 2: return launch_fast_rounds<MODE, 2, LT>(a, s);                 \
      case 3: return launch_fast_rounds<MODE, 3, LT>(a, s);                 \
      case 4: return launch_fast_rounds<MODE, 4, LT>(a, s);                 \
      case 6: return launch_fast_rounds<MODE, 6, LT>(a, s);                 \
      case 8: return launch_fast_rounds<MODE, 8, LT>(a, s);                 \
    }                                                                       \
    return hipErrorInvalidValue;                                            \
  }

// Rotation-only and int8-pack modes of the transposed-gather kernels (no
// code width: BITS is unused by these modes).
#define ORBIT_ROWS_FAST_PLAIN(MODE, LT)                                       \
  template <>                                                               \
  hipError_t launch_fast<MODE, LT>(const RowArgs& a, int, hipStream_t s) {  \
    return launch_fast_rounds<MODE, 4, LT>(a, s);                           \
  }

// Instantiated per (input type, mode) in the rpbh_*.hip files.
template <typename InT, int MODE>
hipError_t launch_mode(const RowArgs& a, int bits, hipStream_t stream);

#define ORBIT_ROWS_QUANT_MODE(InT, MODE)                                     \
  template <>                                                               \
  hipError_t launch_mode<InT, MODE>(const RowArgs& a, int bits, hipStream_t s) { \
    switch (bits) {                                                         \
      case 1: return launch_rounds<InT, MODE, 1>(a, s);                     \
      case 2: return launch_rounds<InT, MODE, 2>(a, s);                     \
      case 3: return launch_rounds<InT, MODE, 3>(a, s);                     \
      case 4: return launch_rounds<InT, MODE, 4>(a, s);                     \
      case 6: return launch_rounds<InT, MODE, 6>(a, s);                     \
      case 8: return launch_rounds<InT, MODE, 8>(a, s);                     \
    }                                                                       \
    return hipErrorInvalidValue;                                            \
  }

#define ORBIT_ROWS_PLAIN_MODE(InT, MODE)                                     \
  template <>                                                               \
  hipError_t launch_mode<InT, MODE>(const RowArgs& a, int, hipStream_t s) {  \
    return launch_rounds<InT, MODE, 4>(a, s);                               \
  }

}  // namespace rows
}  // namespace orbit
