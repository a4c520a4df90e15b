#pragma once
// Decode GEMMs on fp16 matrix cores (gfx950 v_mfma_f32_32x32x16_f16).
//
// OrbitQuant page, Method: because W' = W Pi^T and x' = Pi x, the layer is
// the product of the two quantized factors with no inverse rotation:
//   out[m, n] = s_m r_n (1/K) sum_k ca[ia[m,k]] cw[iw[n,k]]
// (codebooks in N(0,1) units).  The int8 article's load-and-run (section 4)
// is computed in the equal form out = (X Pi^T) (q * scale)^T.
//
// Work layout:
//   * one workgroup = 4 waves = one output tile of TM tokens x TN weight
//     rows; the waves form a 2 x 2 grid, each computing (TM/2) x (TN/2) as
//     WM x WN blocks of 32 x 32 (one wave per SIMD: the 32x32x16 MFMA keeps
//     the matrix core busy from a single wave, the 16x16x32 one does not);
//   * MFMA "A" operand = weight rows (n), "B" operand = tokens (m): lane l
//     feeds row / column l % 32 and holds outputs n = 8 (q/4) + 4 (l/32) +
//     q%4 (q < 16) of token l % 32, i.e. four runs of four consecutive n;
//   * the K loop runs in chunks of KC = 16 * STEPS; within a chunk, lane
//     half g = l / 32 of both operands owns the contiguous k range
//     [g KC/2, (g+1) KC/2), and sub-step s feeds k = g KC/2 + 8 s + 0..7.
//     Both operands use the same assignment, so every dot product is the
//     exact sum over all k while each lane reads one contiguous run of
//     packed codes per row per chunk (16 bytes for 4-bit codes);
//   * codes go straight from global memory to registers (the next chunk is
//     in flight while the current one is multiplied) and are decoded with
//     an LDS table replicated per lane: a code byte and the lane number form
//     the table address in one v_perm, every lane hits its own bank, and a
//     4-bit byte yields two fp16 values per read (a 2-bit byte four);
//   * codebook values are fp16 in N(0,1) units, products accumulate in
//     fp32; s_m r_n / K (+ bias) is applied once in fp32 in the epilogue and
//     the result is rounded once (bf16 nearest even, or kept in fp32).
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "orbit_internal.h"

namespace orbit {
namespace qgemm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  long long M, N, K;
  const uint8_t* a;   // token operand (codes, or fp16 rows for the int8 GEMM)
  const uint8_t* b;   // weight operand (codes, or int8 rows)
  long long lda, ldb; // bytes per row
  const float* s;
  const uint16_t* r_bf16;
  const uint16_t* scale_f16;
  int groups_per_row;
  float inv_k;
  const void* bias;
  int bias_dtype;
  void* out;
  int out_dtype;
  int act;  // orbit_act
  int tiles_m, tiles_n;
  int table_a_offset;  // LDS byte offset of the activation codebook table
  int table_b_offset;  // LDS byte offset of the weight codebook table
  int factor_offset;   // LDS byte offset of the tile's output factors
  uint16_t cent_a[256];
  uint16_t cent_b[256];
};

// Loads from an absolute LDS byte address (the decode tables start at LDS
// offset 0; the kernels use no static LDS).
typedef __attribute__((address_space(3))) const uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) const uint16_t lds_u16_t;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2_t;
__device__ __forceinline__ uint32_t lds_u32(uint32_t a) { return *(lds_u32_t*)(uintptr_t)a; }
__device__ __forceinline__ uint32_t lds_u16(uint32_t a) { return *(lds_u16_t*)(uintptr_t)a; }
__device__ __forceinline__ u32x2 lds_u32x2(uint32_t a) { return *(lds_u32x2_t*)(uintptr_t)a; }

// ---------------------------------------------------------------- operands
// Each operand type knows its chunk (kChunkK), how many bytes a lane loads
// per chunk for one 32-row block, and how to turn sub-step s into a half8.

template <int BITS, int KC>
struct CodeOp {  // packed b-bit codebook indices, LSB-first
  static constexpr int kBits = BITS;
  static constexpr int kChunkK = KC;                   // KC / 16 sub-steps of k = 16
  static constexpr int kBytes = KC * BITS / 16;        // KC / 2 codes per lane per chunk
  static constexpr int kDwords = kBytes / 4;
  static constexpr int kTableBytes = (BITS == 4 || BITS == 2 || BITS == 8) ? 65536 : 16384;
  // LDS reads per sub-step (8 codes): 2-bit bytes give four values, 4-bit
  // bytes and 3- or 6-bit pairs two, 8-bit codes one
  static constexpr int kLookups = BITS == 2 ? 2 : (BITS == 4 || BITS == 3 || BITS == 6) ? 4 : 8;
  // instruction counts per operand and sub-step, for the issue schedule:
  // LDS reads of a gather, VALU work of forming addresses (and of joining
  // 16-bit entries), and global loads per chunk
  static constexpr int kReads = kLookups;
  static constexpr int kValu = (BITS == 2 || BITS == 4) ? kLookups : (BITS == 8 ? 12 : (BITS == 6 ? 2 * kLookups : 3 * kLookups));
  static constexpr int kLoads = (kDwords + 3) / 4;
  uint32_t w[kDwords];

  __device__ __forceinline__ void load(const uint8_t* p) {
    int q = 0;
#pragma unroll
    for (; q + 4 <= kDwords; q += 4) {
      const u32x4 v = *(const u32x4*)(p + 4 * q);
      w[q] = v.x; w[q + 1] = v.y; w[q + 2] = v.z; w[q + 3] = v.w;
    }
    if constexpr (kDwords % 4 == 3) {
      const u32x3 v = *(const u32x3*)(p + 4 * q);
      w[q] = v.x; w[q + 1] = v.y; w[q + 2] = v.z;
    } else if constexpr (kDwords % 4 == 2) {
      const u32x2 v = *(const u32x2*)(p + 4 * q);
      w[q] = v.x; w[q + 1] = v.y;
    } else if constexpr (kDwords % 4 == 1) {
      w[q] = *(const uint32_t*)(p + 4 * q);
    }
  }

  // bits [lo, lo + n) of the lane's code stream (n <= 32)
  __device__ __forceinline__ uint32_t field(int lo, int n) const {
    const int wi = lo >> 5, sh = lo & 31;
    uint32_t v = (sh + n <= 32) ? (w[wi] >> sh) : __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
    return n == 32 ? v : (v & ((1u << n) - 1u));
  }

  // LDS address of lookup l of sub-step s.  `lb` is the lane's base in the
  // decode table (see lane_base); the address takes one v_perm (or a
  // bit-field extract and a shift-or) and no other arithmetic.
  __device__ __forceinline__ uint32_t addr(int s, int l, uint32_t lb) const {
    if constexpr (BITS == 4) {
      // table [byte][64 lanes] of fp16 pairs: addr = base | byte << 8 | lane << 2
      return __builtin_amdgcn_perm(w[s], lb, 0x0c020400u + ((uint32_t)l << 8));
    } else if constexpr (BITS == 2) {
      // table [byte][32 lanes] of fp16 quads: addr = base | byte << 8 | (lane & 31) << 3
      return __builtin_amdgcn_perm(w[s >> 1], lb, 0x0c020400u + ((uint32_t)(2 * (s & 1) + l) << 8));
    } else if constexpr (BITS == 8) {
      // table [byte][64 lanes], fp16 in the low half of each entry
      return __builtin_amdgcn_perm(w[2 * s + (l >> 2)], lb, 0x0c020400u + ((uint32_t)(l & 3) << 8));
    } else if constexpr (BITS == 6) {
      // table [pair of 6-bit indices] of fp16 pairs, one copy for all lanes
      // (4096 entries cannot be replicated per lane: the reads conflict on
      // banks, but two codes per read halve the address work, which bounds
      // the 6-bit decode; measured 10-15 % faster than one code per read).
      // The table sits at a multiple of 16 KB: the address is the pair
      // index shifted into bits 2-13 and OR-ed with the base, one v_bfe and
      // one v_lshl_or (an align and an and for an index across two words).
      // The empty asm keeps that form: folded, the extract and the shift
      // become a shift, an and and an add.  (A lane-permute decode with the
      // 64 values in a register, free of bank conflicts, measured 10 %
      // slower on the video projection.)
      uint32_t p = field(48 * s + 12 * l, 12);
      asm("" : "+v"(p));
      return (p << 2) | lb;
    } else {
      static_assert(BITS == 3, "unsupported width");
      // table [pair of 3-bit indices][64 lanes] of fp16 pairs
      return (field(24 * s + 6 * l, 6) << 8) | lb;
    }
  }

  // the sub-step's eight fp16 values from the addresses of its lookups
  static __device__ __forceinline__ half8 gather(const uint32_t (&a)[kLookups]) {
    uint32_t o[4];
    if constexpr (BITS == 2) {
      const u32x2 q0 = lds_u32x2(a[0]), q1 = lds_u32x2(a[1]);
      o[0] = q0.x; o[1] = q0.y; o[2] = q1.x; o[3] = q1.y;
    } else if constexpr (kLookups == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = lds_u32(a[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = lds_u16(a[2 * j]) | (lds_u16(a[2 * j + 1]) << 16);
    }
    return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
  }

  // The lane's table base: the table's LDS offset (a multiple of 64 KB for
  // the v_perm-addressed tables, of 16 KB for the others) plus the lane's
  // column inside each entry row.
  static __device__ __forceinline__ uint32_t lane_base(uint32_t table_off, uint32_t lane) {
    if constexpr (BITS == 6) return table_off;
    return table_off | (BITS == 2 ? ((lane & 31u) << 3) : (lane << 2));
  }
};

// Chunk length of a pair of code widths: 128 k while the raw codes of both
// operands fit the register budget (2- and 4-bit codes), else 64.
template <int BA, int BB>
struct CodeChunk {
  static constexpr int kK = ((BA == 2 || BA == 4) && (BB == 2 || BB == 4)) ? 128 : 64;
};

// Builds the decode table of a codebook in LDS (256 threads).  Lane-
// replicated tables: every row is 256 bytes (one entry per lane, or per lane
// pair for the 2-bit quads); thread t writes 16-byte piece t % 16 of rows
// t / 16 + 16 k.  The 6-bit pair table has one copy.
template <int BITS>
__device__ __forceinline__ void build_table(char* tab, const uint16_t* cent) {
  if constexpr (BITS == 6) {  // 4096 fp16 pairs: entry i = (c[i % 64], c[i / 64])
    for (int i = threadIdx.x; i < 4096; i += 256)
      *(uint32_t*)(tab + 4 * i) = (uint32_t)cent[i & 63] | ((uint32_t)cent[i >> 6] << 16);
    return;
  }
  constexpr int kRows = BITS == 3 ? 64 : 256;
  const int q = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
  for (int k = 0; k < kRows / 16; ++k) {
    const int r = r0 + 16 * k;
    u32x4 v;
    if constexpr (BITS == 2) {
      const uint32_t lo = (uint32_t)cent[r & 3] | ((uint32_t)cent[(r >> 2) & 3] << 16);
      const uint32_t hi = (uint32_t)cent[(r >> 4) & 3] | ((uint32_t)cent[r >> 6] << 16);
      v = u32x4{lo, hi, lo, hi};
    } else {
      uint32_t e;
      if constexpr (BITS == 4) e = (uint32_t)cent[r & 15] | ((uint32_t)cent[r >> 4] << 16);
      else if constexpr (BITS == 3) e = (uint32_t)cent[r & 7] | ((uint32_t)cent[r >> 3] << 16);
      else e = cent[r];  // 6- and 8-bit: fp16 in the low half
      v = u32x4{e, e, e, e};
    }
    *(u32x4*)(tab + r * 256 + q * 16) = v;
  }
}

struct F16Op {  // fp16 rows (rotated activations of the int8 GEMM)
  static constexpr int kChunkK = 32;  // 2 sub-steps
  static constexpr int kBytes = 32;   // 16 halves per lane per chunk
  u32x4 v[2];
  __device__ __forceinline__ void load(const uint8_t* p) {
    v[0] = *(const u32x4*)p;
    v[1] = *(const u32x4*)(p + 16);
  }
  __device__ __forceinline__ half8 decode(int s, uint32_t) const {
    return __builtin_bit_cast(half8, v[s]);
  }
  static __device__ __forceinline__ uint32_t lane_base(uint32_t, uint32_t) { return 0; }
};

struct I8Op {  // int8 weight rows with an fp16 scale for the chunk's group
  static constexpr int kChunkK = 32;
  static constexpr int kCodeBits = 8;
  typedef u32x4 Raw;  // 16 codes: two sub-steps of 8
  static constexpr int kBytes = 16;  // 16 codes per lane per chunk
  u32x4 v;
  uint32_t scale2;  // the group's fp16 scale in both halves
  __device__ __forceinline__ void load(const uint8_t* p) { v = *(const u32x4*)p; }
  static __device__ __forceinline__ uint32_t lane_base(uint32_t, uint32_t) { return 0; }
  __device__ __forceinline__ half8 decode(int s, uint32_t) const {
    // q + 128 as an unsigned byte u; fp16 bits 0x6400 | u = 1024 + u exactly;
    // subtracting 1152 gives q exactly; one multiply by the scale rounds once
    const uint32_t w0 = (s ? v.z : v.x) ^ 0x80808080u;
    const uint32_t w1 = (s ? v.w : v.y) ^ 0x80808080u;
    const uint32_t mag = 0x64646464u;
    uint32_t h[4];
    h[0] = __builtin_amdgcn_perm(mag, w0, 0x04010400u);
    h[1] = __builtin_amdgcn_perm(mag, w0, 0x04030402u);
    h[2] = __builtin_amdgcn_perm(mag, w1, 0x04010400u);
    h[3] = __builtin_amdgcn_perm(mag, w1, 0x04030402u);
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const half2v sc = __builtin_bit_cast(half2v, scale2);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v q = __builtin_bit_cast(half2v, h[i]) - bias;
      o[i] = __builtin_bit_cast(uint32_t, q * sc);
    }
    return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
  }
};

struct I4Op {  // int4 weight rows (two's-complement nibbles, low nibble
               // first) with an fp16 scale for the chunk's group
  static constexpr int kChunkK = 32;
  static constexpr int kBytes = 8;  // 16 codes per lane per chunk
  static constexpr int kCodeBits = 4;
  typedef uint2 Raw;  // 16 codes: two sub-steps of 8
  uint2 v;
  uint32_t scale2;  // the group's fp16 scale in both halves
  __device__ __forceinline__ void load(const uint8_t* p) { v = *(const uint2*)p; }
  static __device__ __forceinline__ uint32_t lane_base(uint32_t, uint32_t) { return 0; }
  __device__ __forceinline__ half8 decode(int s, uint32_t) const {
    // codes 8 s .. 8 s + 7 of the lane's 16; q + 8 as an unsigned nibble u,
    // spread one per byte in code order, then fp16 bits 0x6400 | u =
    // 1024 + u exactly; subtracting 1032 gives q exactly; one multiply by
    // the scale rounds once
    const uint32_t w = (s ? v.y : v.x) ^ 0x88888888u;
    const uint32_t even = w & 0x0f0f0f0fu;         // codes 0, 2, 4, 6
    const uint32_t odd = (w >> 4) & 0x0f0f0f0fu;   // codes 1, 3, 5, 7
    const uint32_t lo = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // codes 0..3
    const uint32_t hi = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // codes 4..7
    const uint32_t mag = 0x64646464u;
    uint32_t h[4];
    h[0] = __builtin_amdgcn_perm(mag, lo, 0x04010400u);
    h[1] = __builtin_amdgcn_perm(mag, lo, 0x04030402u);
    h[2] = __builtin_amdgcn_perm(mag, hi, 0x04010400u);
    h[3] = __builtin_amdgcn_perm(mag, hi, 0x04030402u);
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    const half2v bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v sc = __builtin_bit_cast(half2v, scale2);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v q = __builtin_bit_cast(half2v, h[i]) - bias;
      o[i] = __builtin_bit_cast(uint32_t, q * sc);
    }
    return __builtin_bit_cast(half8, make_uint4(o[0], o[1], o[2], o[3]));
  }
};

// two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32);
// NaN stays NaN
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.0f); }

__device__ __forceinline__ float load_bias(const GemmArgs& g, long long n) {
  if (!g.bias) return 0.0f;
  if (g.bias_dtype == ORBIT_BF16) return __uint_as_float((uint32_t)((const uint16_t*)g.bias)[n] << 16);
  return ((const float*)g.bias)[n];
}

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0, odd extension; |error| <= 1.5e-7.  Branch
// free: one reciprocal, one exp2 and a Horner polynomial, far below the bf16
// rounding of the output it feeds.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = __builtin_fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, ax, 1.0f));
  float p = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  p *= t;
  const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);  // exp(-x^2)
  return __builtin_copysignf(__builtin_fmaf(-p, e, 1.0f), x);
}

// Output activation applied in fp32 before the output is rounded.
template <int ACT>
__device__ __forceinline__ float act_fn(float y) {
  if constexpr (ACT == ORBIT_ACT_GELU) {
    const float h = 0.5f * y;
    return __builtin_fmaf(h, erf_as7126(y * 0.70710678118654752f), h);  // y/2 (1 + erf(y/sqrt 2))
  } else {
    return y;
  }
}

// Tile order: consecutive workgroups land on different XCDs (round robin), so
// block b is renumbered to give each XCD a contiguous run of tiles, and runs
// are walked in groups of kGroupM token tiles so an XCD shares its operands.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, kGroupM = 4;
  const int total = tiles_m * tiles_n;
  const int full = (total / kXcd) * kXcd;
  int t = b;
  if (b < full) t = (b % kXcd) * (full / kXcd) + b / kXcd;
  const int per_group = kGroupM * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int r = t % per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Issue schedule of one sub-step: NMF MFMAs, each followed by its share of
// the NDS LDS reads, NVA VALU instructions and NVM global loads, so the
// matrix pipe is handed a new MFMA while the previous one is still running.
// With eight or more MFMAs the reads go out behind the first NMF - 4 of
// them: the last four (128 cycles of matrix work) cover the latency of the
// last reads before the next sub-step waits for all of them.
template <int NMF, int NDS, int NVA, int NVM, int K>
__device__ __forceinline__ void issue_slot() {
  constexpr int kReadSlots = NMF >= 8 ? NMF - 4 : NMF;
  constexpr int ds = K < kReadSlots ? NDS * (K + 1) / kReadSlots - NDS * K / kReadSlots : 0;
  constexpr int va = NVA * (K + 1) / NMF - NVA * K / NMF;
  constexpr int vm = NVM * (K + 1) / NMF - NVM * K / NMF;
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
  if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // VMEM read
  if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);  // DS read
  if constexpr (va > 0) __builtin_amdgcn_sched_group_barrier(0x002, va, 0);  // VALU
}
template <int NMF, int NDS, int NVA, int NVM, int... K>
__device__ __forceinline__ void issue_schedule(std::integer_sequence<int, K...>) {
  (issue_slot<NMF, NDS, NVA, NVM, K>(), ...);
}

// Wave grid of a workgroup (4 waves): 2 x 2 for the register-fed kernels,
// 1 x 4 for the staged weight-only kernel (each wave spans all 256 tokens of
// the tile and 64 weight rows, so every decoded weight fragment feeds eight
// MFMAs and no two waves decode the same weights).
template <int KIND>
struct WavesM {
  static constexpr int value = KIND == 2 ? 1 : 2;
};

// s_waitcnt immediate that waits until at most N vector memory loads are in
// flight (vmcnt, bits 3:0 and 15:14) and leaves the LDS/scalar and export
// counters unconstrained.
template <int N>
constexpr int vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

// KIND 0: codebook x codebook; KIND 1: fp16 x int8 or int4 with group scales,
// operands straight from memory; KIND 2: the same product with both operands
// staged through a three-chunk LDS ring (256 x 256 tiles).
// WM token blocks and WN weight blocks of 32 per wave.
template <int KIND, class OpA, class OpB, int WM, int WN>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  extern __shared__ __align__(16) char smem[];
  static_assert(OpA::kChunkK == OpB::kChunkK, "operands must share the chunk");
  constexpr int KC = OpA::kChunkK;
  constexpr int STEPS = KC / 16;
  constexpr int kWM = WavesM<KIND>::value, kWN = 4 / kWM;  // wave grid
  constexpr int TM = 32 * WM * kWM, TN = 32 * WN * kWN;
  static_assert(TM <= 256 && TN <= 512, "the 256 threads stage the factors of TM tokens and TN weight rows");
  constexpr int kNR = (TN + 255) / 256;  // weight-row factors per thread
  const uint32_t lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % kWM, wn = wave / kWM;

  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);

  // The tile's output factors go to LDS next to the tables: s_m / K per
  // token, r_n and the bias per weight row (1, 1 and the bias for the int8
  // GEMM; zero past the end).  Their loads are issued before the tables are
  // built so the two overlap.
  float* const fs = (float*)(smem + g.factor_offset);
  float* const fr = fs + TM;
  float* const fb = fr + TN;
  const int t = threadIdx.x;
  float vs = 1.0f, vr[kNR], vb[kNR];
  {
    const long long m = (long long)tm * TM + t;
    if (KIND == 0 && t < TM) vs = m < g.M ? g.s[m] * g.inv_k : 0.0f;
#pragma unroll
    for (int q = 0; q < kNR; ++q) {
      const int i = t + 256 * q;
      const long long n = (long long)tn * TN + i;
      vr[q] = 1.0f;
      vb[q] = 0.0f;
      if (i < TN) {
        if (KIND == 0) vr[q] = n < g.N ? __uint_as_float((uint32_t)g.r_bf16[n] << 16) : 0.0f;
        vb[q] = n < g.N ? load_bias(g, n) : 0.0f;
      }
    }
  }
  if constexpr (KIND == 0) {
    build_table<OpA::kBits>(smem + g.table_a_offset, g.cent_a);
    if (g.table_a_offset != g.table_b_offset) build_table<OpB::kBits>(smem + g.table_b_offset, g.cent_b);
  }
  if (t < TM) fs[t] = vs;
#pragma unroll
  for (int q = 0; q < kNR; ++q) {
    const int i = t + 256 * q;
    if (i < TN) {
      fr[i] = vr[q];
      fb[i] = vb[q];
    }
  }
  __syncthreads();
  const uint32_t lb_a = OpA::lane_base((uint32_t)g.table_a_offset, lane);
  const uint32_t lb_b = OpB::lane_base((uint32_t)g.table_b_offset, lane);

  const long long m_base = (long long)tm * TM + wm * (32 * WM);
  const long long n_base = (long long)tn * TN + wn * (32 * WN);
  const int r32 = lane & 31, half = lane >> 5;

  // row offsets (rows past the end are clamped; their results are dropped);
  // 32-bit offsets from the operand base keep the loads on one scalar base
  uint32_t oa[WM], ob[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    long long m = m_base + 32 * i + r32;
    m = m < g.M ? m : g.M - 1;
    oa[i] = (uint32_t)(m * g.lda) + (uint32_t)(half * OpA::kBytes);
  }
  uint32_t nrow[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    long long n = n_base + 32 * j + r32;
    n = n < g.N ? n : g.N - 1;
    nrow[j] = (uint32_t)n;
    ob[j] = (uint32_t)(n * g.ldb) + (uint32_t)(half * OpB::kBytes);
  }
  constexpr uint32_t kChunkA = 2u * OpA::kBytes, kChunkB = 2u * OpB::kBytes;

  floatx16 acc[WN][WM];
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.0f;

  const int nchunks = (int)(g.K / KC);  // >= 1
  if constexpr (KIND == 0) {
    // Software pipeline over the sub-steps t of the K loop.  Sub-step t runs
    // its MFMAs on operands gathered during t - 1, gathers the operands of
    // t + 1 from LDS with addresses formed during t - 1, and forms the
    // addresses of t + 2 from the raw codes, so no instruction waits on a
    // result produced just before it.  Raw codes sit in two buffers: chunk
    // c + 2 is loaded into chunk c's buffer as soon as chunk c's last
    // addresses are formed (two sub-steps before its end), a full chunk
    // before it is first read.  Loads past the last chunk re-read the last
    // chunk, and gathers and addresses past the end read valid table
    // entries; neither touches the accumulators.
    OpA ra[2][WM];
    OpB rb[2][WN];
    uint32_t adr_a[WM][OpA::kLookups], adr_b[WN][OpB::kLookups];
    half8 va[2][WM], vb[2][WN];
    const int last = nchunks - 1;
    auto load = [&](int p, int c) {
      c = c < last ? c : last;
#pragma unroll
      for (int i = 0; i < WM; ++i) ra[p][i].load(g.a + oa[i] + (uint32_t)c * kChunkA);
#pragma unroll
      for (int j = 0; j < WN; ++j) rb[p][j].load(g.b + ob[j] + (uint32_t)c * kChunkB);
    };
    auto form = [&](int p, int st) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int l = 0; l < OpA::kLookups; ++l) adr_a[i][l] = ra[p][i].addr(st, l, lb_a);
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int l = 0; l < OpB::kLookups; ++l) adr_b[j][l] = rb[p][j].addr(st, l, lb_b);
    };
    auto gather = [&](int q) {
#pragma unroll
      for (int i = 0; i < WM; ++i) va[q][i] = OpA::gather(adr_a[i]);
#pragma unroll
      for (int j = 0; j < WN; ++j) vb[q][j] = OpB::gather(adr_b[j]);
    };
    auto mma = [&](int q) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[q][j], va[q][i], acc[j][i], 0, 0, 0);
    };
    constexpr int NMF = WM * WN;
    constexpr int NDS = WM * OpA::kReads + WN * OpB::kReads;
    constexpr int NVA = WM * OpA::kValu + WN * OpB::kValu;
    constexpr int NVM = WM * OpA::kLoads + WN * OpB::kLoads;
    using Slots = std::make_integer_sequence<int, NMF>;
    // Each sub-step starts by waiting for all LDS reads issued so far: they
    // are the previous sub-step's gathers, long complete, and one full wait
    // here keeps the MFMAs below free of partial waits (the LDS counter only
    // reaches 15, so a partial wait behind this sub-step's own gathers would
    // stall on them).
    auto chunk = [&](int p, int c) {
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
        if (st == STEPS - 2) load(p, c + 2);
        gather((st + 1) & 1);
        if (st + 2 < STEPS) form(p, st + 2);
        else form(p ^ 1, st + 2 - STEPS);
        mma(st & 1);
        if (st == STEPS - 2) issue_schedule<NMF, NDS, NVA, NVM>(Slots{});
        else issue_schedule<NMF, NDS, NVA, 0>(Slots{});
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    load(0, 0);
    load(1, 1);
    form(0, 0);
    gather(0);
    form(0, 1);
    // Two chunks per trip, buffers 0 and 1 in turn (chunk c in buffer c % 2).
    if constexpr (KC == 64) {
      // K is a multiple of 128 (checked at launch), so 64-k chunks come in
      // pairs.  No odd chunk behind the loop: with one there (the loop's
      // exit feeding a further chunk) the compiler copied every accumulator
      // at each trip for the 3- and 6-bit operands.
      for (int c = 0; c < nchunks; c += 2) {
        chunk(0, c);
        chunk(1, c + 1);
      }
    } else {
      int c = 0;
      for (; c + 1 < nchunks; c += 2) {
        chunk(0, c);
        chunk(1, c + 1);
      }
      if (c < nchunks) chunk(0, c);
    }
  } else if constexpr (KIND == 1) {
    // Raw codes of chunk c + 1 load into the other of two buffers while chunk
    // c is decoded and multiplied.  Decoded token operands are single-
    // buffered: block i is re-decoded for the next sub-step right after its
    // last MFMA of this one; decoded weight operands alternate between two
    // sets, the next set decoded at the start of a sub-step.
    OpA ra0[WM], ra1[WM];
    OpB rb0[WN], rb1[WN];
    auto load_chunk = [&](int c, OpA (&xa)[WM], OpB (&xb)[WN]) {
  #pragma unroll
      for (int i = 0; i < WM; ++i) xa[i].load(g.a + oa[i] + (uint32_t)c * kChunkA);
  #pragma unroll
      for (int j = 0; j < WN; ++j) {
        xb[j].load(g.b + ob[j] + (uint32_t)c * kChunkB);
        if constexpr (KIND == 1) {
          const uint32_t gi = (uint32_t)(c * KC) / 128u;  // group of 128 k
          const uint32_t sc = g.scale_f16[nrow[j] * (uint32_t)g.groups_per_row + gi];
          xb[j].scale2 = sc | (sc << 16);
        }
      }
    };
    half8 av[WM], bv0[WN], bv1[WN];
    auto mfmas = [&](const half8 (&bcur)[WN], int i) {
  #pragma unroll
      for (int j = 0; j < WN; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bcur[j], av[i], acc[j][i], 0, 0, 0);
    };
    // MFMAs of one sub-step with operands (bcur, av) while the next sub-step
    // (xa, xb, ns) is decoded into (av, bnext)
    auto substep_next = [&](const OpA (&xa)[WM], const OpB (&xb)[WN], int ns,
                            const half8 (&bcur)[WN], half8 (&bnext)[WN]) {
  #pragma unroll
      for (int j = 0; j < WN; ++j) bnext[j] = xb[j].decode(ns, lb_b);
  #pragma unroll
      for (int i = 0; i < WM; ++i) {
        mfmas(bcur, i);
        av[i] = xa[i].decode(ns, lb_a);
      }
      // keep the scheduler from hoisting later sub-steps' decodes (and their
      // registers) across this point
      __builtin_amdgcn_sched_barrier(0);
    };
    auto substep_last = [&](const half8 (&bcur)[WN]) {
  #pragma unroll
      for (int i = 0; i < WM; ++i) mfmas(bcur, i);
      __builtin_amdgcn_sched_barrier(0);
    };
    // the STEPS sub-steps of the chunk in (xa, xb); the last one decodes
    // sub-step 0 of the chunk in (ya, yb)
    auto chunk_next = [&](const OpA (&xa)[WM], const OpB (&xb)[WN], const OpA (&ya)[WM],
                          const OpB (&yb)[WN]) {
  #pragma unroll
      for (int s = 0; s < STEPS; s += 2) {
        substep_next(xa, xb, s + 1, bv0, bv1);
        if (s + 2 < STEPS) substep_next(xa, xb, s + 2, bv1, bv0);
        else substep_next(ya, yb, 0, bv1, bv0);
      }
    };
    auto chunk_last = [&](const OpA (&xa)[WM], const OpB (&xb)[WN]) {
  #pragma unroll
      for (int s = 0; s < STEPS; s += 2) {
        substep_next(xa, xb, s + 1, bv0, bv1);
        if (s + 2 < STEPS) substep_next(xa, xb, s + 2, bv1, bv0);
        else substep_last(bv1);
      }
    };

    // the loop body always has a chunk after the one it works on
    load_chunk(0, ra0, rb0);
  #pragma unroll
    for (int i = 0; i < WM; ++i) av[i] = ra0[i].decode(0, lb_a);
  #pragma unroll
    for (int j = 0; j < WN; ++j) bv0[j] = rb0[j].decode(0, lb_b);
    int c = 0;
    for (; c + 2 < nchunks; c += 2) {
      load_chunk(c + 1, ra1, rb1);
      chunk_next(ra0, rb0, ra1, rb1);
      load_chunk(c + 2, ra0, rb0);
      chunk_next(ra1, rb1, ra0, rb0);
    }
    if (c + 1 < nchunks) {  // two chunks left
      load_chunk(c + 1, ra1, rb1);
      chunk_next(ra0, rb0, ra1, rb1);
      chunk_last(ra1, rb1);
    } else {                // one chunk left
      chunk_last(ra0, rb0);
    }
  } else {
    // KIND 2.  Chunks of 64 k; chunk c lives in LDS stage c % 3 while the
    // loads of chunks c + 1 and c + 2 are in flight, and its stage takes
    // chunk c + 3 once every wave has read it.  Loads go global -> LDS
    // directly (16 bytes per lane, written in lane order), so data in flight
    // holds no registers.  Per lane and sub-step s the MFMA k order is
    //   k = 32 half + 8 s + 0..7
    // for both operands, so a lane's k of one chunk are 32 consecutive
    // values.  Stage layout, in 1 KB blocks (one load instruction each), with
    // row r counted inside its block:
    //   tokens (fp16): rows 8b..8b+7 of 128 bytes (64 k); 16-byte piece p of
    //     row r sits at r * 128 + (p ^ ((r / 2) % 8)) * 16 (a lane reads
    //     piece 4 half + s);
    //   weights, int8: rows 16b..16b+15 of 64 bytes; 16-byte unit u at
    //     r * 64 + (u ^ ((r / 4) % 4)) * 16 (a lane reads unit 2 half + s/2,
    //     two sub-steps at once);
    //   weights, int4: rows 32b..32b+31 of 32 bytes; 16-byte unit u at
    //     r * 32 + (u ^ ((r / 8) % 2)) * 16 (a lane reads unit half once per
    //     chunk, all four sub-steps);
    //   group scales: 256 dwords, tile row t at dword t, the aligned dword
    //     that holds the fp16 scale of (row, chunk's group).
    // LDS serves a 16-byte read for 16 lanes (16 consecutive rows) at a
    // time across 256 bytes; the XOR swizzles put those 16 rows in 16
    // different 16-byte bank groups, while each load instruction still
    // covers whole rows of the chunk.
    // The loads are issued with inline assembly and waited for explicitly
    // (vmcnt, then a bare s_barrier): they have no register results, and the
    // compiler, which cannot tell the stages apart, would otherwise wait for
    // every load in flight before each LDS read.
    static_assert(WM == 8 && WN == 2 && kWM == 1, "the staged loop is laid out for 256 x 256 tiles, 1 x 4 waves");
    constexpr int kCK = 64;
    constexpr bool kI4 = OpB::kCodeBits == 4;
    constexpr int kBRow = kCK * OpB::kCodeBits / 8;   // weight bytes per row per chunk
    constexpr int kABytes = TM * kCK * 2;              // 32 KB
    constexpr int kBBytes = TN * kBRow;                // 16 or 8 KB
    constexpr int kSBytes = TN * 4;                    // scale dwords
    constexpr int kStage = kABytes + kBBytes + kSBytes;
    constexpr int kALoads = kABytes / 1024 / 4;        // per thread per chunk
    constexpr int kBLoads = kBBytes / 1024 / 4;
    constexpr int kLoads = kALoads + kBLoads + 1;
    static_assert(kStage % 16 == 0, "stages stay 16-byte aligned");
    const int nch = (int)(g.K / kCK);                  // >= 2 (K % 128 == 0)
    const int last = nch - 1;
    const uint32_t wv = __builtin_amdgcn_readfirstlane((uint32_t)wave);

    // global sources of this thread's loads (rows past the end are clamped:
    // valid memory, results dropped)
    uint32_t ga[kALoads], gb[kBLoads];
#pragma unroll
    for (int q = 0; q < kALoads; ++q) {
      const int blk = q * 4 + wave, r8 = lane >> 3;
      long long m = (long long)tm * TM + 8 * blk + r8;
      m = m < g.M ? m : g.M - 1;
      const int f = ((8 * blk + r8) >> 1) & 7;
      ga[q] = (uint32_t)(m * g.lda) + (uint32_t)((((int)lane & 7) ^ f) * 16);
    }
#pragma unroll
    for (int q = 0; q < kBLoads; ++q) {
      const int blk = q * 4 + wave;
      int r, u;
      if constexpr (kI4) {
        r = 32 * blk + (lane >> 1);
        u = ((int)lane & 1) ^ ((lane >> 4) & 1);
      } else {
        r = 16 * blk + (lane >> 2);
        u = ((int)lane & 3) ^ ((lane >> 4) & 3);
      }
      long long n = (long long)tn * TN + r;
      n = n < g.N ? n : g.N - 1;
      gb[q] = (uint32_t)(n * g.ldb) + (uint32_t)(u * 16);
    }
    // scale element of (tile row t, group 0); the dword holding element e
    // starts at byte 2 (e & ~1), and element e is its half e & 1
    uint32_t gs;
    {
      long long n = (long long)tn * TN + t;
      n = n < g.N ? n : g.N - 1;
      gs = (uint32_t)n * (uint32_t)g.groups_per_row;
    }
    // loads chunk c (clamped to the last chunk) into the stage of chunk cs
    auto issue = [&](int cs, int c) {
      c = c < last ? c : last;
      const uint32_t st = (uint32_t)(cs % 3) * kStage;
#pragma unroll
      for (int q = 0; q < kALoads; ++q)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(st + (q * 4 + wv) * 1024u), "v"(ga[q] + (uint32_t)c * (kCK * 2)), "s"(g.a)
                     : "memory", "m0");
#pragma unroll
      for (int q = 0; q < kBLoads; ++q)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(st + kABytes + (q * 4 + wv) * 1024u), "v"(gb[q] + (uint32_t)c * kBRow), "s"(g.b)
                     : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                   :: "s"(st + kABytes + kBBytes + wv * 256u), "v"(((gs + (uint32_t)(c >> 1)) & ~1u) * 2u),
                      "s"(g.scale_f16)
                   : "memory", "m0");
    };
    // this lane's LDS read offsets inside a stage
    const uint32_t xa = (r32 >> 1) & 7;
    const uint32_t a_base = (uint32_t)(wm * 4 * WM + (r32 >> 3)) * 1024u + (r32 & 7) * 128u;
    uint32_t a_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a_off[s] = a_base + (((uint32_t)(4 * half + s) ^ xa) << 4);
    uint32_t b_off[2];
    constexpr uint32_t kBBlock = kI4 ? 1024u : 2048u;  // LDS bytes per 32 weight rows
    if constexpr (kI4) {
      const uint32_t x4 = (r32 >> 3) & 1;
      b_off[0] = (uint32_t)kABytes + (uint32_t)(wn * WN) * 1024u + r32 * 32u + (((uint32_t)half ^ x4) << 4);
      b_off[1] = b_off[0];
    } else {
      const uint32_t r16 = r32 & 15, x8 = (r16 >> 2) & 3;
      const uint32_t b_base = (uint32_t)kABytes + (uint32_t)(wn * 2 * WN + (r32 >> 4)) * 1024u + r16 * 64u;
#pragma unroll
      for (int v = 0; v < 2; ++v) b_off[v] = b_base + (((uint32_t)(2 * half + v) ^ x8) << 4);
    }
    const uint32_t s_off = (uint32_t)(kABytes + kBBytes) + (uint32_t)(wn * 32 * WN + r32) * 4u;
    uint32_t s_par[WN];  // parity of the lane's scale element at group 0
#pragma unroll
    for (int j = 0; j < WN; ++j) s_par[j] = (nrow[j] * (uint32_t)g.groups_per_row) & 1u;

    // Operands in flight: token blocks and decoded weight blocks of two
    // sub-steps (sub-step s of a chunk uses set s & 1), raw weights of the
    // chunk (int8: unit r holds sub-steps 2r and 2r + 1; int4: unit 0 holds
    // all four) and the group scales of the chunk.
    half8 av[2][WM], bv[2][WN];
    u32x4 braw[2][WN];
    uint32_t sc[WN];
    auto read_a = [&](int set, const char* st, int s) {
#pragma unroll
      for (int i = 0; i < WM; ++i) av[set][i] = *(const half8*)(st + a_off[s] + i * 4096);
    };
    auto read_raw = [&](int unit, const char* st) {
#pragma unroll
      for (int j = 0; j < WN; ++j) braw[unit][j] = *(const u32x4*)(st + b_off[unit] + j * kBBlock);
    };
    auto read_scale = [&](const char* st, int c) {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t dw = *(const uint32_t*)(st + s_off + j * 128);
        const uint32_t h16 = (dw >> (16 * ((s_par[j] + (uint32_t)(c >> 1)) & 1u))) & 0xffffu;
        sc[j] = h16 | (h16 << 16);
      }
    };
    auto decode = [&](int set, int s) {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        OpB op;
        if constexpr (kI4) op.v = make_uint2(braw[0][j][s], 0u);
        else op.v = braw[s >> 1][j];
        op.scale2 = sc[j];
        bv[set][j] = op.decode(kI4 ? 0 : (s & 1), 0);
      }
    };
    auto mma = [&](int set) {
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int i = 0; i < WM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[set][j], av[set][i], acc[j][i], 0, 0, 0);
    };
    // Issue order of a sub-step: each MFMA followed by up to R LDS reads and
    // V VALU instructions, so the reads and the decode of the next sub-step
    // go out while the matrix pipe works on this one.
    auto interleave = [&](auto r_, auto v_) {
      constexpr int R = decltype(r_)::value, V = decltype(v_)::value;
#pragma unroll
      for (int q = 0; q < WM * WN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int kV = kI4 ? 3 : 2;  // decode VALU per MFMA slot

    // Chunk c + 1 must be complete before the last sub-step of chunk c reads
    // it: every chunk issues the same kLoads loads, and chunk c + 2's are the
    // only ones issued after chunk c + 1's, so waiting until at most kLoads
    // are in flight completes it.  The wait also drains this wave's LDS reads
    // (lgkmcnt 0), after which the barrier means every wave is done reading
    // chunk c's stage, which then takes chunk c + 3.  The empty asm
    // statements keep the compiler from moving memory accesses across the
    // barrier.
    auto sync = [&](auto n_) {
      __builtin_amdgcn_s_waitcnt(vm_wait<decltype(n_)::value>() & ~(15 << 8));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    sync(std::integral_constant<int, 2 * kLoads>{});  // chunk 0 complete
    read_scale(smem, 0);
    read_raw(0, smem);
    read_a(0, smem, 0);
    decode(0, 0);
    // sub-steps 0-2 of chunk c: MFMAs on set s & 1 while the token blocks of
    // sub-step s + 1 are read and its weight blocks decoded (int8: the raw
    // unit of sub-steps 2 and 3 is read during sub-step 0)
    auto first3 = [&](const char* st) {
      mma(0);
      if constexpr (!kI4) read_raw(1, st);
      read_a(1, st, 1);
      decode(1, 1);
      interleave(std::integral_constant<int, 1>{}, std::integral_constant<int, kV>{});
      mma(1);
      read_a(0, st, 2);
      decode(0, 2);
      interleave(std::integral_constant<int, 1>{}, std::integral_constant<int, kV>{});
      mma(0);
      read_a(1, st, 3);
      decode(1, 3);
      interleave(std::integral_constant<int, 1>{}, std::integral_constant<int, kV>{});
    };
    // The last chunk runs the same body: its reads of "chunk last + 1" read
    // a stage that holds a re-read of the last chunk (valid LDS, values
    // unused), so the loop has one body and no tail.
    for (int c = 0; c < nch; ++c) {
      const char* const st = smem + (c % 3) * kStage;
      const char* const sn = smem + ((c + 1) % 3) * kStage;
      first3(st);
      // sub-step 3: chunk c + 1 complete and chunk c's stage free; its loads
      // go out, chunk c + 1's scales, first raw unit and first token blocks
      // are read, and its first weight blocks are decoded in the second half
      // of the MFMAs
      sync(std::integral_constant<int, kLoads>{});
      issue(c + 3, c + 3);
      read_scale(sn, c + 1);
      read_raw(0, sn);
      read_a(0, sn, 0);
      mma(1);
      decode(0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * WN + WM, 0);
#pragma unroll
      for (int q = 0; q < WM * WN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q >= WM * WN / 2) __builtin_amdgcn_sched_group_barrier(0x002, 2 * kV + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the trailing re-reads must land before the epilogue reuses the ring
    __builtin_amdgcn_s_waitcnt(vm_wait<0>());
  }

  // epilogue: block (j, i) of lane l holds weight rows
  // n_base + 32 j + 8 qq + 4 half + 0..3 (qq < 4) of token m_base + 32 i + r32.
  // The factors come from LDS.  A wave whose outputs lie inside the matrix,
  // with row length and output pointer aligned for 8/16-byte stores, takes
  // the vector path with no per-element checks.
  const float* const ws = fs + wm * (32 * WM) + r32;
  const float* const wr = fr + wn * (32 * WN) + 4 * half;
  const float* const wb = fb + wn * (32 * WN) + 4 * half;
  float sm[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) sm[i] = ws[32 * i];
  // the whole output path, for one activation (uniform choice below)
  auto finish = [&](auto actc) {
    constexpr int ACT = decltype(actc)::value;
    const bool f32_out = g.out_dtype != ORBIT_BF16;
    const bool fast = (g.N & 3) == 0 && ((uintptr_t)g.out & 15) == 0 && m_base + 32 * WM <= g.M &&
                      n_base + 32 * WN <= g.N;
    auto epi = [&](auto f32c) {
      constexpr bool F32 = decltype(f32c)::value;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const long long n0 = n_base + 32 * j + 8 * qq + 4 * half;
          const float4 cf = *(const float4*)(wr + 32 * j + 8 * qq);
          const float4 cb = *(const float4*)(wb + 32 * j + 8 * qq);
          const float cfv[4] = {cf.x, cf.y, cf.z, cf.w}, cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            const long long m = m_base + 32 * i + r32;
            float y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) y[q] = act_fn<ACT>(__builtin_fmaf(acc[j][i][4 * qq + q], sm[i] * cfv[q], cbv[q]));
            if constexpr (F32) {
              *(float4*)((float*)g.out + m * g.N + n0) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
              u32x2 w;
              w.x = pack_bf16x2(y[0], y[1]);
              w.y = pack_bf16x2(y[2], y[3]);
              *(u32x2*)((uint16_t*)g.out + m * g.N + n0) = w;
            }
          }
        }
      }
    };
    // Whole tile inside a bf16 output with 16-byte aligned rows: the tile is
    // staged in LDS (over the decode tables, which the K loop no longer needs)
    // and written out row by row, 16 bytes per lane, so each output row of the
    // tile leaves as whole cache lines instead of 16-byte pieces of 32 rows.
    // The condition is the same for every wave of the workgroup.
    const bool staged = !f32_out && (g.N & 7) == 0 && ((uintptr_t)g.out & 15) == 0 &&
                        (long long)(tm + 1) * TM <= g.M && (long long)(tn + 1) * TN <= g.N;
    if (staged) {
      constexpr int kRow = TN * 2 + 16;  // padded LDS row: 2-way bank conflicts at most
      __syncthreads();                   // every wave is done with the tables
      const int lm = wm * (32 * WM) + r32, ln = wn * (32 * WN) + 4 * half;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float4 cf = *(const float4*)(wr + 32 * j + 8 * qq);
          const float4 cb = *(const float4*)(wb + 32 * j + 8 * qq);
          const float cfv[4] = {cf.x, cf.y, cf.z, cf.w}, cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            float y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) y[q] = act_fn<ACT>(__builtin_fmaf(acc[j][i][4 * qq + q], sm[i] * cfv[q], cbv[q]));
            u32x2 w;
            w.x = pack_bf16x2(y[0], y[1]);
            w.y = pack_bf16x2(y[2], y[3]);
            *(u32x2*)(smem + (lm + 32 * i) * kRow + (ln + 32 * j + 8 * qq) * 2) = w;
          }
        }
      }
      __syncthreads();
      constexpr int kChunks = TN * 2 / 16;  // 16-byte pieces per tile row
      char* const out0 = (char*)g.out + ((long long)tm * TM * g.N + (long long)tn * TN) * 2;
#pragma unroll 4
      for (int q = t; q < TM * kChunks; q += 256) {
        const int row = q / kChunks, c = q - row * kChunks;
        const u32x4 v = *(const u32x4*)(smem + row * kRow + c * 16);
        // streaming stores: the output is not read again by this kernel
        // (measured 1-2 % on the image layer)
        __builtin_nontemporal_store(v, (u32x4*)(out0 + (long long)row * g.N * 2 + c * 16));
      }
      return;
    }
    if (fast) {
      if (f32_out) epi(std::true_type{});
      else epi(std::false_type{});
      return;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long long n = n_base + 32 * j + 8 * qq + 4 * half + q;
          if (n >= g.N) continue;
          const float cf = wr[32 * j + 8 * qq + q], cb = wb[32 * j + 8 * qq + q];
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            const long long m = m_base + 32 * i + r32;
            if (m >= g.M) continue;
            const float y = act_fn<ACT>(__builtin_fmaf(acc[j][i][4 * qq + q], sm[i] * cf, cb));
            if (f32_out) ((float*)g.out)[m * g.N + n] = y;
            else ((uint16_t*)g.out)[m * g.N + n] = f32_to_bf16_rne(y);
          }
        }
      }
    }
  };
  if (g.act == ORBIT_ACT_GELU) finish(std::integral_constant<int, ORBIT_ACT_GELU>{});
  else finish(std::integral_constant<int, ORBIT_ACT_NONE>{});
}

template <int KIND, class OpA, class OpB, int WM, int WN>
hipError_t launch_tile(GemmArgs& g, int lds, hipStream_t stream) {
  if (KIND == 0 && OpA::kChunkK == 64 && g.K % 128 != 0) return hipErrorInvalidValue;  // chunk pairs
  constexpr int kWM = WavesM<KIND>::value, kWN = 4 / kWM;
  constexpr int TM = 32 * WM * kWM, TN = 32 * WN * kWN;
  g.tiles_m = (int)((g.M + TM - 1) / TM);
  g.tiles_n = (int)((g.N + TN - 1) / TN);
  const long long tiles = (long long)g.tiles_m * g.tiles_n;
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  // LDS: the decode tables (reused by the staged bf16 epilogue, which needs
  // TM rows of TN * 2 + 16 bytes), then the tile's output factors
  const int tile_bytes = TM * (TN * 2 + 16);
  g.factor_offset = lds > tile_bytes ? lds : tile_bytes;  // a multiple of 16
  lds = g.factor_offset + (TM + 2 * TN) * (int)sizeof(float);
  auto kern = gemm_kernel<KIND, OpA, OpB, WM, WN>;
  static LaunchCache cache;
  hipError_t e = prepare_launch(cache, (const void*)kern, 256, lds, nullptr);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), lds, stream, g);
  return hipGetLastError();
}

// Picks the tile: large tiles when there are enough of them to fill the
// 256 compute units, smaller ones otherwise.  Codes wider than 4 bits (and
// 3-bit codes) hold more raw bits and table addresses per operand, so their
// widest wave tile is 4 x 2 blocks instead of 4 x 3, and 2 x 2 for the
// pairs whose registers do not fit 4 x 2 (both operands 6- or 8-bit, or
// 8-bit tokens with 3-bit weights).  Products of at least three tiles per
// compute unit take 2 x 8 (or 2 x 6) wave tiles where the registers allow
// them: 6-bit tokens and 2-bit weights.
template <int KIND, class OpA, class OpB>
hipError_t launch_shape(GemmArgs& g, int lds, hipStream_t stream) {
  auto tiles = [&](int tm, int tn) { return ((g.M + tm - 1) / tm) * ((g.N + tn - 1) / tn); };
  constexpr bool kNarrow = KIND == 1 || OpA::kChunkK == 128;
  if constexpr (kNarrow) {
    if constexpr (KIND == 0) {
      if constexpr (OpB::kBits == 2) {
        // 2-bit weights (four values per read): the 2 x 8 wave tile halves
        // the token-code reads per MFMA against 4 x 3 and fits the registers
        if (tiles(128, 512) >= 768) return launch_tile<KIND, OpA, OpB, 2, 8>(g, lds, stream);
      }
    }
    if (tiles(256, 192) >= 192) return launch_tile<KIND, OpA, OpB, 4, 3>(g, lds, stream);
  } else if constexpr (!(OpA::kLookups + OpB::kLookups >= 16 || (OpA::kBits == 8 && OpB::kBits == 3))) {
    // the operand with the costlier decode gets the shorter side of the wave
    // tile: each of its blocks is decoded once per sub-step and feeds one
    // MFMA per block of the other operand
    if constexpr (KIND == 0 && OpA::kValu > OpB::kValu) {
      if constexpr (OpA::kBits == 6) {
        // 6-bit tokens: their pair table's reads conflict on banks, so wider
        // wave tiles feed each of them to eight (2 x 8) or six (2 x 6) MFMAs.
        // With 4-bit weights the 4 x 4 tile comes first: 32 LDS lookups per
        // 16 MFMAs against 40 on 2 x 8, and the lookup count, not the
        // conflicts, bounds the loop (four copies of the pair table, one per
        // lane class, left the time unchanged; 4 x 4 measured 5 % faster on
        // the video projection).  With 2-bit weights 4 x 4 spills.
        if constexpr (OpB::kBits == 4) {
          if (tiles(256, 256) >= 768) return launch_tile<KIND, OpA, OpB, 4, 4>(g, lds, stream);
        }
        if (tiles(128, 512) >= 768) return launch_tile<KIND, OpA, OpB, 2, 8>(g, lds, stream);
        if (tiles(128, 384) >= 768) return launch_tile<KIND, OpA, OpB, 2, 6>(g, lds, stream);
      }
      if (tiles(128, 256) >= 192) return launch_tile<KIND, OpA, OpB, 2, 4>(g, lds, stream);
    } else {
      if (tiles(256, 128) >= 192) return launch_tile<KIND, OpA, OpB, 4, 2>(g, lds, stream);
    }
  }
  if (tiles(128, 128) >= 128) return launch_tile<KIND, OpA, OpB, 2, 2>(g, lds, stream);
  return launch_tile<KIND, OpA, OpB, 1, 1>(g, lds, stream);
}

// LDS layout of the two decode tables.  Tables addressed through v_perm
// (2-, 4- and 8-bit codes, 64 KB each) must start at a multiple of 64 KB,
// so a 64 KB table goes first; 3- and 6-bit tables (16 KB) only need 16 KB
// alignment.  A shared codebook uses one table.
template <int BA, int BB>
hipError_t launch_codes(GemmArgs& g, hipStream_t stream, bool same_table) {
  constexpr int KC = CodeChunk<BA, BB>::kK;
  using OpA = CodeOp<BA, KC>;
  using OpB = CodeOp<BB, KC>;
  const int tab_a = OpA::kTableBytes, tab_b = OpB::kTableBytes;
  int lds;
  if (same_table) {
    g.table_a_offset = 0;
    g.table_b_offset = 0;
    lds = tab_a;
  } else if (tab_a >= tab_b) {
    g.table_a_offset = 0;
    g.table_b_offset = tab_a;
    lds = tab_a + tab_b;
  } else {
    g.table_b_offset = 0;
    g.table_a_offset = tab_b;
    lds = tab_a + tab_b;
  }
  return launch_shape<0, OpA, OpB>(g, lds, stream);
}

// Defined (and instantiated) in qgemm_a<BA>.hip, one translation unit per
// activation width so the kernels compile in parallel.
template <int BA>
hipError_t launch_codes_b(GemmArgs& g, int bb, hipStream_t stream, bool same);

#define ORBIT_DEFINE_LAUNCH_CODES_B(BA)                                          \
  template <>                                                                   \
  hipError_t launch_codes_b<BA>(GemmArgs & g, int bb, hipStream_t stream, bool same) { \
    switch (bb) {                                                               \
      case 2: return launch_codes<BA, 2>(g, stream, false);                     \
      case 3: return launch_codes<BA, 3>(g, stream, false);                     \
      case 4: return launch_codes<BA, 4>(g, stream, same && BA == 4);           \
      case 6: return launch_codes<BA, 6>(g, stream, false);                     \
      case 8: return launch_codes<BA, 8>(g, stream, same && BA == 8);           \
    }                                                                           \
    return hipErrorInvalidValue;                                                \
  }

hipError_t launch_int8(GemmArgs& g, hipStream_t stream);
hipError_t launch_int4(GemmArgs& g, hipStream_t stream);

}  // namespace qgemm
}  // namespace orbit
