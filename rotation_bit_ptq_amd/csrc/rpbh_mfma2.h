// Rotate + quantize with the block Hadamard on the matrix cores, codes packed
// in registers: bf16 rows, h = 128 or 256, d = 1024 .. 4096 (one wave per
// row) or 8192, 12288, 16384 (four waves per row), codebook modes
// (activations, weights) and the fp16 rotation.
//
// OrbitQuant page, Method: x' = blkdiag(H_h D_i) P_pi x.  In Sylvester order
// H_h is the Kronecker product of H_2 over the log2(h) bits of the position
// inside a block, so any split of those bits into factors gives the same
// transform.  Here the split is chosen so that every lane ends up holding
// consecutive positions, which lets it pack its codes in registers and
// store them straight to memory:
//   * the two lowest bits b0 b1 index the rows of the MFMA's A operand
//     (four rows per block) and come out as the four accumulator values
//     e = 0..3 of a lane: H_4 over them is two register stages;
//   * five bits index the MFMA's contraction (k = 0..31): H_32 is the
//     product with the +-1 operand B, exactly as bf16 x bf16 -> fp32;
//   * for h = 256 the remaining bit b2 picks one of two MFMA calls on the
//     same lanes (m = 0, 1): H_2 over it is one more register stage.
// A unit of work is 4 blocks: 512 positions for h = 128 (one A operand, two
// MFMAs for the two 16-column halves of H_32), 1024 for h = 256 (two A
// operands, four MFMAs).  Lane l = 16 kq + r16 gathers A row r16 = 4 (block
// in unit) + t' with contraction slots 8 kq + j, and receives output rows
// 4 kq + e of column r16 (+16 for the second half): block kq of the unit,
// positions 4 j' + e (h = 128) or 8 j' + 4 m + e (h = 256), j' = r16 or
// r16 + 16, i.e. 4 or 8 consecutive positions.
//
// Per row, one of two forms brings each lane's A operands into LDS order:
//   * scatter (activations on a permuting rotation with a plan): each lane
//     writes the bf16 values it loaded, sign-flipped by D, straight to the
//     operand slots the plan's scatter section names, so every operand is
//     16 contiguous bytes and one 16-byte read;
//   * gather (everything else): the row lands once in LDS (at address 0,
//     with a 16-byte pad after every 64 coordinates up to 12288
//     coordinates, so that the strided reads of an identity permutation
//     spread over the banks), and each lane gathers its operand pairs with
//     two 16-bit reads from the plan's offset words (or words built from pi
//     and the signs), which also carry the sign flips D (XOR into bits 15
//     and 31).
#pragma once

#include <type_traits>

#include "rpbh_mfma.h"

namespace orbit {
namespace rows {
namespace m2 {

typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint16_t lds_u16_st_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// The two 32 x 16 halves of H_32 as each lane's B operands (lane l = 16 kq
// + r16 holds rows 8 kq .. 8 kq + 7 of columns r16 and r16 + 16, Sylvester
// entries (-1)^popcount(i & j) as bf16), built at compile time: two 16-byte
// loads per wave instead of the entries' arithmetic.
struct H32Table {
  uint32_t w[64][8];
};
constexpr uint32_t h32_bf16(int i, int j) { return (__builtin_popcount(i & j) & 1) ? 0xBF80u : 0x3F80u; }
constexpr H32Table make_h32_table() {
  H32Table t{};
  for (int lane = 0; lane < 64; ++lane) {
    const int r16 = lane & 15, kq = lane >> 4;
    for (int q = 0; q < 4; ++q) {
      const int k0 = 8 * kq + 2 * q;
      t.w[lane][q] = h32_bf16(k0, r16) | (h32_bf16(k0 + 1, r16) << 16);
      t.w[lane][4 + q] = h32_bf16(k0, r16 + 16) | (h32_bf16(k0 + 1, r16 + 16) << 16);
    }
  }
  return t;
}
static __device__ const H32Table kH32Table = make_h32_table();

// Positions per unit and A operands per unit, by h = 32 G.
template <int G> struct Unit;
template <> struct Unit<4> { static constexpr int kPos = 512, kOps = 1; };
template <> struct Unit<8> { static constexpr int kPos = 1024, kOps = 2; };

// LDS byte address of coordinate p of the row (the row starts at 0).
template <bool kPad>
__host__ __device__ constexpr uint32_t row_addr(int p) {
  return 2u * (uint32_t)p + (kPad ? 16u * (uint32_t)(p >> 6) : 0u);
}
// Rows with a pad: up to 12288 coordinates (the 15-bit byte offsets of the
// plan's words then stay below 2^15).
__host__ __device__ constexpr bool padded(int d) { return d <= 12288; }
__host__ __device__ constexpr int row_lds_bytes(int d) { return padded(d) ? 2 * d + 16 * (d / 64) : 2 * d; }

// Permuted index k of slot j (0..7) of operand o for lane (kq, r16).
template <int G>
__host__ __device__ constexpr int slot_k(int o, int kq, int r16, int j) {
  if (G == 4) return 512 * o + 128 * (r16 >> 2) + 32 * kq + 4 * j + (r16 & 3);
  return 1024 * (o >> 1) + 256 * (r16 >> 2) + 64 * kq + 8 * j + 4 * (o & 1) + (r16 & 3);
}

// y_k = D_k x[pi(k)] as two bf16 in one register: the word holds the LDS
// byte offsets of the pair in bits 0-14 and 16-30 and their sign flips in
// bits 15 and 31.  Four VALU per pair: the two offsets, the merge and the
// sign XOR (v_bitop3).
__device__ __forceinline__ uint32_t gather_pair(uint32_t w) {
  ushort2v p;
  p.x = *(lds_cu16_t*)(uintptr_t)(w & 0x7fffu);
  p.y = *(lds_cu16_t*)(uintptr_t)((w >> 16) & 0x7fffu);
  return __builtin_bit_cast(uint32_t, p) ^ (w & 0x80008000u);
}

// Offset words of operands o0 .. o0 + NO - 1 for this lane: from the plan
// (16 bytes per lane and operand), or built from pi and the signs.
template <int G, int NO, bool kPad>
__device__ __forceinline__ void load_words(const RowArgs& a, int o0, int lane,
                                           uint32_t (&w)[NO][4]) {
  if (a.mfma_words) {  // uniform
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const u32x4 v = *(const u32x4*)(a.mfma_words + 4 * (64 * (o0 + i) + lane));
      w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
    }
    return;
  }
  const int kq = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int i = 0; i < NO; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = slot_k<G>(o0 + i, kq, r16, 2 * q), k1 = slot_k<G>(o0 + i, kq, r16, 2 * q + 1);
      const uint32_t s0 = (a.sign_bits[k0 >> 5] >> (k0 & 31)) & 1u;
      const uint32_t s1 = (a.sign_bits[k1 >> 5] >> (k1 & 31)) & 1u;
      w[i][q] = row_addr<kPad>(a.perm[k0]) | (s0 << 15) | (row_addr<kPad>(a.perm[k1]) << 16) | (s1 << 31);
    }
  }
}

// Scatters one loaded dword (bf16 x[i], x[i + 1]) to the operand slots
// that need it: the plan's scatter word holds the two slots' LDS byte
// offsets in bits 0-14 and 16-30 and the sign flips D of their permuted
// indices in bits 15 and 31.  Three VALU per pair (the sign XOR and the two
// offsets); the high half goes out with ds_write_b16_d16_hi.
__device__ __forceinline__ void scatter_pair(uint32_t x, uint32_t w) {
  const uint32_t y = x ^ (w & 0x80008000u);
  *(lds_u16_st_t*)(uintptr_t)(w & 0x7fffu) = (uint16_t)y;
  *(lds_u16_st_t*)(uintptr_t)((w >> 16) & 0x7fffu) = (uint16_t)(y >> 16);
}

// Redefines the offset words at the top of every row (an empty asm, in
// place: no copy), so the compiler cannot unpack them once outside the row
// loop, which would take three times their registers.
template <int N>
__device__ __forceinline__ void opaque_words(uint32_t (&w)[N][4]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(w[i][q]));
}

// Stores n code bytes (n = 1..8) at p from the packed value v (LSB first),
// with the widest stores the alignment allows (p is aligned to the largest
// power of two dividing n, except for 3 bytes: byte stores).
template <int N>
__device__ __forceinline__ void store_code_bytes(uint8_t* p, uint64_t v) {
  if constexpr (N == 1) {
    *p = (uint8_t)v;
  } else if constexpr (N == 2) {
    *(uint16_t*)p = (uint16_t)v;
  } else if constexpr (N == 3) {
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
  } else if constexpr (N == 4) {
    *(uint32_t*)p = (uint32_t)v;
  } else if constexpr (N == 6) {
    uint16_t* q = (uint16_t*)p;
    q[0] = (uint16_t)v;
    q[1] = (uint16_t)(v >> 16);
    q[2] = (uint16_t)(v >> 32);
  } else {
    static_assert(N == 8, "code run of 1, 2, 3, 4, 6 or 8 bytes");
    *(u32x2*)p = u32x2{(uint32_t)v, (uint32_t)(v >> 32)};
  }
}

// The units of one row handled by this wave: units u0 .. u0 + NU - 1 of the
// row held in LDS, in steps of 8 values per lane (two MFMAs): a whole unit
// for h = 128 (two runs of 4 positions), one half of a unit for h = 256
// (one run of 8).  The gathers of unit u + 1 are in flight during the steps
// of unit u, and the grid-cell reads of step s while step s + 1 multiplies;
// the codes of step s are packed and stored during step s + 1.
template <int MODE, int BITS, int G, int NU, int D, bool kX, bool kSc>
__device__ __forceinline__ void units(const RowArgs& a, long long row, int u0,
                                      uint32_t (&w)[NU * Unit<G>::kOps][4],
                                      const bf16x8& hb0, const bf16x8& hb1, float cell_a,
                                      uint32_t gbias, int lane) {
  extern __shared__ __align__(16) char smem[];
  constexpr bool kQuant = MODE != kRotF16;
  constexpr int NO = Unit<G>::kOps;
  constexpr int SPU = NO;               // steps per unit
  constexpr int NS = NU * SPU;          // steps of this wave's share of the row
  constexpr int RUN = 4 * NO;           // consecutive positions per run
  constexpr int NR = 8 / RUN;           // runs per step
  const int r16 = lane & 15, kq = lane >> 4;
  const float top = kMagic + (float)(a.cells - 1);
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // first position of run r of step s: block kq of unit s / SPU, column
  // j' = r16 + 16 hf with hf = r (h = 128) or s % SPU (h = 256)
  auto run_pos = [&](int st, int r) {
    const int u = st / SPU, hf = SPU == 1 ? r : st % SPU;
    return Unit<G>::kPos * (u0 + u) + (32 * G) * kq + RUN * (r16 + 16 * hf);
  };
  // Pipelined values alternate between two register sets by the parity of
  // their unit or step (the loop is unrolled, so the indices are constants
  // and nothing is copied from one set to the other): the gathered pairs of
  // unit u in pr[u & 1]; the values of step s and their grid cells in
  // uu[s & 1] and g[s & 1], compared and packed during step s + 1.
  uint32_t pr[2][NO][4];
  auto gather = [&](int u) {
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if constexpr (kSc) {  // the row was scattered into operand order
        const u32x4 v = *(const u32x4*)(smem + 16 * (64 * (NO * (u0 + u) + o) + lane));
        pr[u & 1][o][0] = v.x; pr[u & 1][o][1] = v.y; pr[u & 1][o][2] = v.z; pr[u & 1][o][3] = v.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) pr[u & 1][o][q] = gather_pair(w[NO * u + o][q]);
      }
    }
  };
  gather(0);
  float uu[2][8];
  GridCell g[2][8];
#pragma unroll
  for (int st = 0; st <= NS; ++st) {
    float v[8];  // run r: v[RUN r + c] is position run_pos(st, r) + c
    if (st < NS) {
      // a new unit: the next unit's gathers
      if (st % SPU == 0 && st / SPU + 1 < NU) gather(st / SPU + 1);
      const int ub = (st / SPU) & 1;
      bf16x8 av[NO];
#pragma unroll
      for (int o = 0; o < NO; ++o)
        av[o] = __builtin_bit_cast(bf16x8, make_uint4(pr[ub][o][0], pr[ub][o][1], pr[ub][o][2], pr[ub][o][3]));
      floatx4 y0, y1;
      if constexpr (G == 4) {  // both halves of H_32 on the one operand
        y0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], hb0, zero, 0, 0, 0);
        y1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], hb1, zero, 0, 0, 0);
      } else {                 // half st % 2 of H_32 on both operands (m = 0, 1)
        const bf16x8& hb = (st % 2) ? hb1 : hb0;
        y0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], hb, zero, 0, 0, 0);
        y1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1], hb, zero, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = y0[e];
        v[4 + e] = y1[e];
      }
    }
    if (kQuant && st > 0) {  // the codes of step st - 1
      using Packed = std::conditional_t<(RUN * BITS > 32), uint64_t, uint32_t>;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        Packed packed = 0;
        if constexpr (RUN == 4 && BITS == 4) {
          // a tree of three shift-ors (the compiler's own form of the chain
          // took four: two shifts, a shift-or and an or3); the empty asm
          // keeps the pairs from being re-associated
          uint32_t id[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const GridCell& gc = g[(st - 1) & 1][RUN * r + c];
            id[c] = (uint32_t)(gc.base + (gc.t < uu[(st - 1) & 1][RUN * r + c] ? 1 : 0));
          }
          uint32_t lo = (id[1] << 4) | id[0], hi = (id[3] << 4) | id[2];
          asm volatile("" : "+v"(lo), "+v"(hi));
          packed = (hi << 8) | lo;
        } else {
#pragma unroll
          for (int c = RUN - 1; c >= 0; --c) {
            const GridCell& gc = g[(st - 1) & 1][RUN * r + c];
            const int idx = gc.base + (gc.t < uu[(st - 1) & 1][RUN * r + c] ? 1 : 0);
            packed = (Packed)(packed << BITS) | (Packed)idx;
          }
        }
        uint8_t* out = a.idx_out + (size_t)row * ((size_t)D * BITS / 8) +
                       (size_t)run_pos(st - 1, r) * BITS / 8;
        store_code_bytes<RUN * BITS / 8>(out, packed);
      }
    }
    if (st < NS) {
      group_stages<4>(v[0], v[1], v[2], v[3]);
      group_stages<4>(v[4], v[5], v[6], v[7]);
      if constexpr (G == 8) {  // H_2 over the MFMA call m (position bit b2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[e], y = v[4 + e];
          v[e] = x + y;
          v[4 + e] = x - y;
        }
      }
      if constexpr (!kQuant) {  // fp16 x'
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          uint32_t h2[RUN / 2];
#pragma unroll
          for (int c = 0; c < RUN / 2; ++c)
            h2[c] = (uint32_t)f32_to_f16_rne(v[RUN * r + 2 * c] * a.inv_sqrt_h) |
                    ((uint32_t)f32_to_f16_rne(v[RUN * r + 2 * c + 1] * a.inv_sqrt_h) << 16);
          uint16_t* out = a.xrot_f16 + (size_t)row * D + run_pos(st, r);
          if constexpr (RUN == 4) *(u32x2*)out = u32x2{h2[0], h2[1]};
          else *(u32x4*)out = u32x4{h2[0], h2[1], h2[2], h2[3]};
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uu[st & 1][c] = v[c];
          g[st & 1][c] = *(const GridCell*)(smem + grid_addr(v[c], cell_a, a.gb, top, gbias));
        }
        if constexpr (kX) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            float* out = a.xrot_f32 + (size_t)row * D + run_pos(st, r);
#pragma unroll
            for (int c = 0; c < RUN; c += 4)
              *(float4*)(out + c) = make_float4(v[RUN * r + c] * a.inv_sqrt_h, v[RUN * r + c + 1] * a.inv_sqrt_h,
                                                v[RUN * r + c + 2] * a.inv_sqrt_h, v[RUN * r + c + 3] * a.inv_sqrt_h);
          }
        }
      }
    }
    // one step at a time: hoisting later gathers would hold their registers
    __builtin_amdgcn_sched_barrier(0);
  }
}

// W waves per row (1 for d <= 4096, 4 beyond), NU units per wave.  The
// occupancy hint is the register budget the instances meet without spills
// (hipcc's resource report): four waves per SIMD up to 3072 coordinates
// per wave for h = 128 (2048 with 6-bit codes) and 2048 for h = 256, three
// beyond; two for the debug copy.  G: h = 32 G; NU: units per wave.
constexpr int waves_hint(int G, int NU, int BITS, bool x) {
  return x ? 2 : ((G == 4 ? 512 : 1024) * NU <= (G == 8 || BITS == 6 ? 2048 : 3072) ? 4 : 3);
}

// kSc: the row is scattered into operand order through the plan's scatter
// section (a permuting rotation with a plan) and each operand is one
// 16-byte read; otherwise the lanes gather their operands from the row.
template <int MODE, int BITS, int G, int NU, int W, bool kX, bool kSc>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(waves_hint(G, NU, BITS, kX))))
void kernel(RowArgs a) {
  static_assert(MODE == kAct || MODE == kWeight || MODE == kRotF16, "codebook modes and fp16 x'");
  static_assert(G == 4 || G == 8, "h = 128 or 256");
  constexpr bool kQuant = MODE != kRotF16;
  constexpr int NO = Unit<G>::kOps;
  constexpr int D = Unit<G>::kPos * NU * W;
  constexpr bool kPad = padded(D);
  constexpr int NT = 64 * W;            // threads per row
  constexpr int NCH = D / 8 / NT;       // 16-byte row chunks per thread
  static_assert(D / 8 % NT == 0, "whole chunks per thread");
  static_assert(NCH == NU * NO, "one offset word set per 16-byte chunk or per operand");
  constexpr uint32_t kRed = (uint32_t)row_lds_bytes(D);      // four wave sums (W = 4)
  constexpr uint32_t kGrid = kRed + 16u;                      // the grid table
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  float* const red = (float*)(smem + kRed);
  const uint32_t gbias = a.grid_bias + kGrid;

  const u32x4* hp = (const u32x4*)kH32Table.w[lane];
  const bf16x8 hb0 = __builtin_bit_cast(bf16x8, hp[0]), hb1 = __builtin_bit_cast(bf16x8, hp[1]);
  // the row first (global loads retire in order: the waits for the words
  // and the grid below then also cover the row)
  u32x4 pre[NCH];
  auto load = [&](long long rr) {
    const u32x4* src = (const u32x4*)((const char*)a.in + (size_t)rr * D * 2);
#pragma unroll
    for (int i = 0; i < NCH; ++i) pre[i] = __builtin_nontemporal_load(src + t + NT * i);
  };
  long long row = blockIdx.x;
  load(row < a.rows ? row : a.rows - 1);
  uint32_t w[NU * NO][4];
  if constexpr (kSc) {  // scatter words of this thread's chunks (plan order)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const u32x4 v = *(const u32x4*)(a.scatter_words + 4 * (t + NT * i));
      w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
    }
  } else {
    load_words<G, NU * NO, kPad>(a, NO * NU * wave, lane, w);
  }
  // The quantizer compares the unscaled rotated values v (u = alpha v)
  // with the row's thresholds t / alpha, rewritten in the grid each row
  // from a copy of the grid's thresholds kept after it, and the cell of v
  // is fma(v, alpha a, b): one multiply per row instead of one per
  // coordinate.  Decisions can differ from those on u = alpha v only within
  // a few float32 ulps of a threshold.
  GridCell* const grid = (GridCell*)(smem + kGrid);
  float* const thr = (float*)(smem + kGrid + a.grid_bytes);
  // grids of at most one cell per thread (the usual case: 32 cells for
  // 4-bit codes) keep the thread's threshold in a register, so the per-row
  // rewrite waits on no LDS read
  const bool thr_in_reg = a.cells <= NT;
  float thr_r = 0.0f;
  if constexpr (kQuant) {
    build_grid(a, smem + kGrid);
    __syncthreads();
    for (int c = t; c < a.cells; c += NT) thr[c] = grid[c].t;
    if (thr_in_reg && t < a.cells) thr_r = grid[t].t;
  }
  auto rescale = [&](float inv) {
    if (thr_in_reg) {
      if (t < a.cells) grid[t].t = thr_r * inv;
    } else {
      for (int c = t; c < a.cells; c += NT) grid[c].t = thr[c] * inv;
    }
  };

  for (; row < a.rows; row += gridDim.x) {
    opaque_words(w);
    float ssx = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if constexpr (kQuant) ssx = RowRegs<uint16_t, 1>::chunk_sumsq(pre[i], ssx);
      if constexpr (kSc) {
        const uint32_t x[4] = {pre[i].x, pre[i].y, pre[i].z, pre[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) scatter_pair(x[q], w[i][q]);
      } else {
        const int c = t + NT * i;  // chunk c: coordinates 8 c .. 8 c + 7
        *(u32x4*)(smem + row_addr<kPad>(8 * c)) = pre[i];
      }
    }
    if (row + gridDim.x < a.rows) load(row + gridDim.x);
    float alpha = 0.0f;
    if constexpr (W == 1) {
      if constexpr (kQuant) {
        float inv;
        alpha = row_alpha_inv<MODE>(a, wave_sum(ssx), row, lane, inv);
        rescale(inv);
      }
      __syncthreads();  // the row and the row's thresholds are in LDS
    } else {
      if constexpr (kQuant) {
        const float ws = wave_sum(ssx);
        if (lane == 0) red[wave] = ws;
      }
      __syncthreads();  // the row and the wave sums are in LDS
      if constexpr (kQuant) {
        float inv;
        alpha = row_alpha_inv<MODE>(a, (red[0] + red[1]) + (red[2] + red[3]), row, t, inv);
        rescale(inv);
        __syncthreads();  // the row's thresholds are in LDS
      }
    }
    units<MODE, BITS, G, NU, D, kX, kSc>(a, row, NU * wave, w, hb0, hb1, alpha * a.ga, gbias, lane);
    __syncthreads();  // every lane has gathered before the next row lands
  }
}

template <int MODE, int BITS, int G, int NU, int W, bool kX, bool kSc>
hipError_t launch_typed(const RowArgs& a, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  constexpr int D = Unit<G>::kPos * NU * W;
  // the row, four wave sums, the grid and a copy of its thresholds
  const int lds = row_lds_bytes(D) + 16 + a.grid_bytes + a.grid_bytes / 2;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  auto kern = kernel<MODE, BITS, G, NU, W, kX, kSc>;
  static LaunchCache cache;
  int per_cu = 1;
  e = prepare_launch(cache, (const void*)kern, 64 * W, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * W), lds, stream, a);
  return hipGetLastError();
}

template <int MODE, int BITS, int G, bool kX, bool kSc>
hipError_t launch_dd(const RowArgs& a, hipStream_t stream) {
  constexpr int P = Unit<G>::kPos;
  switch (a.d) {
    case 1024: return launch_typed<MODE, BITS, G, 1024 / P, 1, kX, kSc>(a, stream);
    case 2048: return launch_typed<MODE, BITS, G, 2048 / P, 1, kX, kSc>(a, stream);
    case 3072: if constexpr (3072 % P == 0) return launch_typed<MODE, BITS, G, 3072 / P, 1, kX, kSc>(a, stream);
               break;
    case 4096: return launch_typed<MODE, BITS, G, 4096 / P, 1, kX, kSc>(a, stream);
    case 8192: return launch_typed<MODE, BITS, G, 8192 / P / 4, 4, kX, kSc>(a, stream);
    case 12288: return launch_typed<MODE, BITS, G, 12288 / P / 4, 4, kX, kSc>(a, stream);
    case 16384: return launch_typed<MODE, BITS, G, 16384 / P / 4, 4, kX, kSc>(a, stream);
  }
  return hipErrorInvalidValue;
}

// The scatter form serves the online activation quantizer (the other modes
// run offline or keep the gather form).
template <int MODE, int BITS, int G, bool kX>
hipError_t launch_d(const RowArgs& a, hipStream_t stream) {
  if constexpr (MODE == kAct) {
    if (a.scatter_words) return launch_dd<MODE, BITS, G, kX, true>(a, stream);
  }
  return launch_dd<MODE, BITS, G, kX, false>(a, stream);
}


// ---- blocks of 512 .. 4096 coordinates (the full RHT of the rotation
// ablation, h = d) on rows of 2048 or 4096 coordinates, one wave per row.
// In Sylvester order H_h = H_{h/128} (x) H_128 over the position's bits
// above and below bit 7.  The h = 128 factor runs as above (units of four
// 128-blocks, block kq of unit u in lane group kq), which leaves each lane
// all 8 NU values of its positions, NU = d / 512 units.  The factor over the
// 128-block index q = 4 u + kq (log2(h / 128) bits) then runs as register
// stages over the unit bits below log2(h / 512), and two butterflies across
// lanes for the kq bits (lane bits 5 and 4): v_permlane32_swap and
// v_permlane16_swap exchange the halves (rows of 16) of two registers, after
// which an add and a subtract give both registers' butterflies, with the
// two registers' halves transposed: afterwards, register u of lane l holds
// unit U and lane L with U's bit PA equal to lane bit 5 and L's bit 5 equal
// to u's bit PA (and likewise bit PB with lane bit 4), PA and PB being the
// two top unit bits.
template <int MODE, int BITS, int NU, int LOGH, bool kX>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kX ? 2 : (NU == 8 ? 2 : 3))))
void big_kernel(RowArgs a) {
  static_assert(MODE == kAct || MODE == kWeight || MODE == kRotF16, "codebook modes and fp16 x'");
  static_assert((NU == 4 || NU == 8) && LOGH >= 9 && LOGH <= 12 && (1 << LOGH) <= 512 * NU,
                "blocks of 512 .. 4096 on rows of 2048 or 4096");
  constexpr bool kQuant = MODE != kRotF16;
  constexpr int D = 512 * NU;
  constexpr int UB = LOGH - 9;               // unit bits inside a block
  constexpr int PA = NU == 8 ? 2 : 1, PB = PA - 1;
  constexpr uint32_t kRed = (uint32_t)row_lds_bytes(D);
  constexpr uint32_t kGrid = kRed + 16u;
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const uint32_t gbias = a.grid_bias + kGrid;
  const u32x4* hp = (const u32x4*)kH32Table.w[lane];
  const bf16x8 hb0 = __builtin_bit_cast(bf16x8, hp[0]), hb1 = __builtin_bit_cast(bf16x8, hp[1]);
  u32x4 pre[NU];
  auto load = [&](long long rr) {
    const u32x4* src = (const u32x4*)((const char*)a.in + (size_t)rr * D * 2);
#pragma unroll
    for (int i = 0; i < NU; ++i) pre[i] = __builtin_nontemporal_load(src + lane + 64 * i);
  };
  long long row = blockIdx.x;
  load(row < a.rows ? row : a.rows - 1);
  uint32_t w[NU][4];
  load_words<4, NU, true>(a, 0, lane, w);
  GridCell* const grid = (GridCell*)(smem + kGrid);
  float* const thr = (float*)(smem + kGrid + a.grid_bytes);
  if constexpr (kQuant) {
    build_grid(a, smem + kGrid);
    __syncthreads();
    for (int c = lane; c < a.cells; c += 64) thr[c] = grid[c].t;
  }
  const float top = kMagic + (float)(a.cells - 1);
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};

  for (; row < a.rows; row += gridDim.x) {
    opaque_words(w);
    float ssx = 0.0f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      if constexpr (kQuant) ssx = RowRegs<uint16_t, 1>::chunk_sumsq(pre[i], ssx);
      *(u32x4*)(smem + row_addr<true>(8 * (lane + 64 * i))) = pre[i];
    }
    if (row + gridDim.x < a.rows) load(row + gridDim.x);
    float alpha = 0.0f;
    if constexpr (kQuant) {
      alpha = row_alpha<MODE, true>(a, wave_sum(ssx), row, lane);
      const float inv = 1.0f / alpha;
      for (int c = lane; c < a.cells; c += 64) grid[c].t = thr[c] * inv;
    }
    __syncthreads();  // the row and the row's thresholds are in LDS
    // the h = 128 factor, unit by unit: v[u][4 hf + e] is position
    // 512 u + 128 kq + 4 (r16 + 16 hf) + e
    float v[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      uint32_t pr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) pr[q] = gather_pair(w[u][q]);
      const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(pr[0], pr[1], pr[2], pr[3]));
      const floatx4 y0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb0, zero, 0, 0, 0);
      const floatx4 y1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb1, zero, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[u][e] = y0[e];
        v[u][4 + e] = y1[e];
      }
      group_stages<4>(v[u][0], v[u][1], v[u][2], v[u][3]);
      group_stages<4>(v[u][4], v[u][5], v[u][6], v[u][7]);
    }
    __syncthreads();  // every lane has gathered: the row buffer is free
    // the unit bits inside a block, in registers
#pragma unroll
    for (int b = 0; b < UB; ++b)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (!(u & (1 << b)))
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float x = v[u][c], y = v[u | (1 << b)][c];
            v[u][c] = x + y;
            v[u | (1 << b)][c] = x - y;
          }
    // the kq bits across lanes: lane bit 5 with units paired on bit PA,
    // then lane bit 4 with units paired on bit PB
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (!(u & (1 << PA)))
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[u][c]),
                                                          __float_as_uint(v[u | (1 << PA)][c]), false, false);
          const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
          v[u][c] = x + y;
          v[u | (1 << PA)][c] = x - y;
        }
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (!(u & (1 << PB)))
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[u][c]),
                                                          __float_as_uint(v[u | (1 << PB)][c]), false, false);
          const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
          v[u][c] = x + y;
          v[u | (1 << PB)][c] = x - y;
        }
    // position of register (u, hf)'s run in this lane after the exchanges
    auto run_pos = [&](int u, int hf) {
      const int U = (u & ~((1 << PA) | (1 << PB))) | (((lane >> 5) & 1) << PA) | (((lane >> 4) & 1) << PB);
      const int kqL = 2 * ((u >> PA) & 1) + ((u >> PB) & 1);
      return 512 * U + 128 * kqL + 4 * (r16 + 16 * hf);
    };
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int p = run_pos(u, hf);
        if constexpr (!kQuant) {
          const uint32_t h0 = (uint32_t)f32_to_f16_rne(v[u][4 * hf] * a.inv_sqrt_h) |
                              ((uint32_t)f32_to_f16_rne(v[u][4 * hf + 1] * a.inv_sqrt_h) << 16);
          const uint32_t h1 = (uint32_t)f32_to_f16_rne(v[u][4 * hf + 2] * a.inv_sqrt_h) |
                              ((uint32_t)f32_to_f16_rne(v[u][4 * hf + 3] * a.inv_sqrt_h) << 16);
          *(u32x2*)(a.xrot_f16 + (size_t)row * D + p) = u32x2{h0, h1};
        } else {
          const float cell_a = alpha * a.ga;
          uint32_t packed = 0;
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const float x = v[u][4 * hf + e];
            const GridCell g = *(const GridCell*)(smem + grid_addr(x, cell_a, a.gb, top, gbias));
            packed = (packed << BITS) | (uint32_t)(g.base + (g.t < x ? 1 : 0));
          }
          store_code_bytes<4 * BITS / 8>(a.idx_out + (size_t)row * ((size_t)D * BITS / 8) + (size_t)p * BITS / 8,
                                         packed);
          if constexpr (kX) {
            float* out = a.xrot_f32 + (size_t)row * D + p;
            *(float4*)out = make_float4(v[u][4 * hf] * a.inv_sqrt_h, v[u][4 * hf + 1] * a.inv_sqrt_h,
                                        v[u][4 * hf + 2] * a.inv_sqrt_h, v[u][4 * hf + 3] * a.inv_sqrt_h);
          }
        }
      }
    }
  }
}

template <int MODE, int BITS, int NU, int LOGH, bool kX>
hipError_t launch_big_typed(const RowArgs& a, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int lds = row_lds_bytes(512 * NU) + 16 + a.grid_bytes + a.grid_bytes / 2;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  auto kern = big_kernel<MODE, BITS, NU, LOGH, kX>;
  static LaunchCache cache;
  int per_cu = 1;
  e = prepare_launch(cache, (const void*)kern, 64, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64), lds, stream, a);
  return hipGetLastError();
}

template <int MODE, int BITS, bool kX>
hipError_t launch_big(const RowArgs& a, hipStream_t stream) {
  if (a.d == 2048) {
    switch (a.h) {
      case 512: return launch_big_typed<MODE, BITS, 4, 9, kX>(a, stream);
      case 1024: return launch_big_typed<MODE, BITS, 4, 10, kX>(a, stream);
      case 2048: return launch_big_typed<MODE, BITS, 4, 11, kX>(a, stream);
    }
  } else if (a.d == 4096) {
    switch (a.h) {
      case 512: return launch_big_typed<MODE, BITS, 8, 9, kX>(a, stream);
      case 1024: return launch_big_typed<MODE, BITS, 8, 10, kX>(a, stream);
      case 2048: return launch_big_typed<MODE, BITS, 8, 11, kX>(a, stream);
      case 4096: return launch_big_typed<MODE, BITS, 8, 12, kX>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace m2

// Which rows the packed-code kernels take (bf16 input): h = 128 or 256 and
// d = 1024, 2048, 3072 (h = 128 or 256 with 3072 % 1024 == 0), 4096, 8192,
// 12288 or 16384; codes of 2, 4, 6 or 8 bits, and 3 bits when h = 256 (a
// lane's run of 8 codes is 3 whole bytes); or the fp16 rotation.
// Blocks of 512 .. 4096 coordinates on rows of 2048 or 4096 (big_kernel):
// codes of 2, 4, 6 or 8 bits, or the fp16 rotation.
inline bool m2_big_takes(int d, int h, int bits, bool rot_f16) {
  if (!(d == 2048 || d == 4096) || h < 512 || h > d) return false;
  return rot_f16 || bits == 2 || bits == 4 || bits == 6 || bits == 8;
}

inline bool m2_takes(int d, int h, int bits, bool rot_f16) {
  if (h != 128 && h != 256) return false;
  const bool dok = d == 1024 || d == 2048 || d == 3072 || d == 4096 || d == 8192 || d == 12288 || d == 16384;
  if (!dok) return false;
  if (rot_f16) return true;
  return bits == 2 || bits == 4 || bits == 6 || bits == 8 || (bits == 3 && h == 256);
}

template <int MODE, int G>
hipError_t launch_m2(const RowArgs& a, int bits, hipStream_t stream);
template <int MODE>
hipError_t launch_m2_big(const RowArgs& a, int bits, hipStream_t stream);

#define ORBIT_ROWS_M2_BIG(MODE)                                                              \
  template <>                                                                              \
  hipError_t launch_m2_big<MODE>(const RowArgs& a, int bits, hipStream_t s) {              \
    const bool x = MODE == kAct && a.xrot_f32 != nullptr;                                  \
    switch (bits) {                                                                        \
      case 2: return x ? m2::launch_big<MODE, 2, true>(a, s) : m2::launch_big<MODE, 2, false>(a, s); \
      case 4: return x ? m2::launch_big<MODE, 4, true>(a, s) : m2::launch_big<MODE, 4, false>(a, s); \
      case 6: return x ? m2::launch_big<MODE, 6, true>(a, s) : m2::launch_big<MODE, 6, false>(a, s); \
      case 8: return x ? m2::launch_big<MODE, 8, true>(a, s) : m2::launch_big<MODE, 8, false>(a, s); \
    }                                                                                      \
    return hipErrorInvalidValue;                                                           \
  }

#define ORBIT_ROWS_M2_BIG_ROT                                                                \
  template <>                                                                              \
  hipError_t launch_m2_big<kRotF16>(const RowArgs& a, int, hipStream_t s) {                \
    return m2::launch_big<kRotF16, 4, false>(a, s);                                        \
  }

#define ORBIT_ROWS_M2(MODE, G)                                                               \
  template <>                                                                              \
  hipError_t launch_m2<MODE, G>(const RowArgs& a, int bits, hipStream_t s) {               \
    const bool x = MODE == kAct && a.xrot_f32 != nullptr;                                  \
    switch (bits) {                                                                        \
      case 2: return x ? m2::launch_d<MODE, 2, G, true>(a, s) : m2::launch_d<MODE, 2, G, false>(a, s); \
      case 3: if constexpr (G == 8) return x ? m2::launch_d<MODE, 3, G, true>(a, s) : m2::launch_d<MODE, 3, G, false>(a, s); \
              break;                                                                       \
      case 4: return x ? m2::launch_d<MODE, 4, G, true>(a, s) : m2::launch_d<MODE, 4, G, false>(a, s); \
      case 6: return x ? m2::launch_d<MODE, 6, G, true>(a, s) : m2::launch_d<MODE, 6, G, false>(a, s); \
      case 8: return x ? m2::launch_d<MODE, 8, G, true>(a, s) : m2::launch_d<MODE, 8, G, false>(a, s); \
    }                                                                                      \
    return hipErrorInvalidValue;                                                           \
  }

#define ORBIT_ROWS_M2_ROT(G)                                                                 \
  template <>                                                                              \
  hipError_t launch_m2<kRotF16, G>(const RowArgs& a, int, hipStream_t s) {                 \
    return m2::launch_d<kRotF16, 4, G, false>(a, s);                                       \
  }

}  // namespace rows
}  // namespace orbit
