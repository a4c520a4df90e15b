// Rotate + quantize with the block Hadamard on the matrix cores: bf16 rows,
// h = 32 G (G = 2, 4, 8: h = 64, 128, 256), d = 512 C (C = 2, 4, 6, 8),
// codebook modes (activations and weights) and the fp16 rotation.
//
// OrbitQuant page, Method: x' = blkdiag(H_h D_i) P_pi x.  In Sylvester order
// H_h = H_G (x) H_32: with position p = 32 t + r of a block (t < G groups of
// r < 32), y_p = sum_t' H_G[t][t'] sum_r' H_32[r][r'] z_{32 t' + r'} for the
// signed, permuted block z.  The inner sum over r' is a matrix product
// Z (groups x 32) . H_32, run as v_mfma_f32_16x16x32_bf16 pairs: 16 groups
// (16 / G blocks of G groups) times the two 32 x 16 halves of H_32.  Both
// factors are exact in bf16 (z is a bf16 input with its sign flipped, H_32
// is +-1) and the products accumulate in fp32, so the result matches the
// fp32 butterflies up to rounding order.  The lane layout of that
// instruction gives lane l the 4 consecutive groups 4 (l / 16) .. + 3 of the
// pair, at columns r and r + 16: H_G is register stages over those 4
// groups (two stages for G = 4, one for G = 2) and, for G = 8, one more
// stage between lanes l and l ^ 16.  Against the butterfly kernels this
// removes the bf16 widening, five of the log2(h) butterfly stages and the
// LDS transpose from every coordinate.
//
// Per row (one wave, as in rows_kernel): the row lands once in the wave's
// LDS buffer; each lane gathers 8 coordinates per MFMA pair (its A fragment:
// permuted positions 8 (lane / 16) .. + 7 of group (lane % 16) % 4 of block
// 4 c + (lane % 16) / 4) and flips their sign bits with masks kept in
// registers; codes go to a per-wave byte buffer in position order and leave
// as packed 16-code words, like the other row kernels.
#pragma once

#include "rpbh_impl.h"

namespace orbit {
namespace rows {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const uint16_t lds_cu16_t;

__device__ __forceinline__ uint32_t lds_read_u16(uint32_t addr) {
  return *(lds_cu16_t*)(uintptr_t)addr;
}

// Sylvester-order Hadamard entry (-1)^popcount(i & j) as a bf16 bit pattern.
__device__ __forceinline__ uint16_t hadamard_bf16(int i, int j) {
  return (__builtin_popcount(i & j) & 1) ? 0xBF80u : 0x3F80u;
}

// Butterflies over a lane's four consecutive groups: span 1, and span 2
// when a block has 4 or more groups.
template <int G>
__device__ __forceinline__ void group_stages(float& v0, float& v1, float& v2, float& v3) {
  const float a0 = v0 + v1, a1 = v0 - v1, a2 = v2 + v3, a3 = v2 - v3;
  if constexpr (G == 2) {
    v0 = a0; v1 = a1; v2 = a2; v3 = a3;
  } else {
    v0 = a0 + a2;
    v2 = a0 - a2;
    v1 = a1 + a3;
    v3 = a1 - a3;
  }
}

// The H_32 column halves as MFMA B operands: lane holds k = 8 kq + j of
// column r16 (first half) and r16 + 16 (second half).
__device__ __forceinline__ void hadamard32_operands(int r16, int kq, bf16x8& hb0, bf16x8& hb1) {
  uint32_t hw0[4], hw1[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k0 = 8 * kq + 2 * q;
    hw0[q] = hadamard_bf16(k0, r16) | ((uint32_t)hadamard_bf16(k0 + 1, r16) << 16);
    hw1[q] = hadamard_bf16(k0, r16 + 16) | ((uint32_t)hadamard_bf16(k0 + 1, r16 + 16) << 16);
  }
  hb0 = __builtin_bit_cast(bf16x8, make_uint4(hw0[0], hw0[1], hw0[2], hw0[3]));
  hb1 = __builtin_bit_cast(bf16x8, make_uint4(hw1[0], hw1[1], hw1[2], hw1[3]));
}

// Gather offsets and signs of pairs c0 .. c0 + NP - 1.  Pair c covers
// positions 512 c .. + 511 (16 / G whole blocks), group rho = 16 c +
// (position % 512) / 32 being A row rho % 16; element j of the lane's
// fragment is permuted position k = 512 c + 32 r16 + 8 kq + j, for any G.
// y_k = D_k x[pi(k)] is the bf16 at byte 2 pi(k) of the row buffer with its
// sign bit flipped when D_k < 0.  Elements 2 q and 2 q + 1 share word q: the
// low and high halves hold their byte offsets (below 2^15 for d <= 16384)
// and, in bits 15 and 31, their sign flips, so the word masked with
// 0x80008000 is the XOR that applies D to the gathered pair.
// kIdent: pi is the identity (the caller's promise): the words hold only
// the signs, and each fragment is 16 contiguous bytes of the row.
// With the rotation's plan the words of a random pi are read from it
// (16 bytes per lane and pair) instead of being built from pi and the signs.
template <int NP, bool kIdent>
__device__ __forceinline__ void pair_offsets(const RowArgs& a, int c0, int r16, int kq,
                                             uint32_t (&off)[NP][4]) {
  if (!kIdent && a.mfma_words) {  // uniform
    const int lane = 16 * kq + r16;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const u32x4 w = *(const u32x4*)(a.mfma_words + 4 * (64 * (c0 + i) + lane));
      off[i][0] = w.x; off[i][1] = w.y; off[i][2] = w.z; off[i][3] = w.w;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int k0 = 512 * (c0 + i) + 32 * r16 + 8 * kq;
    const uint32_t sw = a.sign_bits[k0 >> 5] >> (k0 & 31);  // 8 signs (k0 % 8 == 0)
    int p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (!kIdent) {
      const i32x4 p0 = *(const i32x4*)(a.perm + k0), p1 = *(const i32x4*)(a.perm + k0 + 4);
      p[0] = p0.x; p[1] = p0.y; p[2] = p0.z; p[3] = p0.w;
      p[4] = p1.x; p[5] = p1.y; p[6] = p1.z; p[7] = p1.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      off[i][q] = ((uint32_t)p[2 * q] * 2u) | ((uint32_t)p[2 * q + 1] << 17) |
                  (((sw >> (2 * q)) & 1u) << 15) | (((sw >> (2 * q + 1)) & 1u) << 31);
  }
}

// Pairs c0 .. c0 + NP - 1 of one row in the buffer at rbuf: gather, H_32 on
// the matrix cores, H_G, then the codes (a byte per position at cbuf) or,
// for kRotF16, fp16 x' (two bytes per position at cbuf); kX also writes
// fp32 x' to xr.  The gathers of pair i + 1 and the grid-cell reads of
// pair i are in flight while pair i is multiplied.
template <int MODE, int G, int NP, bool kX, bool kIdent>
__device__ __forceinline__ void mfma_pairs(const RowArgs& a, uint32_t rbuf, uint32_t cbuf,
                                           int c0, uint32_t (&off)[NP][4],
                                           const bf16x8& hb0, const bf16x8& hb1, float alpha,
                                           float* xr, int lane) {
  // the kernel's dynamic LDS: with the array's known alignment the 8-byte
  // grid cells are read as one ds_read_b64 rather than two 4-byte reads
  extern __shared__ __align__(16) char smem[];
  constexpr bool kQuant = MODE != kRotF16;
  const int r16 = lane & 15, kq = lane >> 4;
  const float top = kMagic + (float)(a.cells - 1);
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // (the empty asm keeps the offsets packed: unpacked once outside the row
  // loop they would take twice the registers)
  auto gather = [&](int i, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
    if constexpr (kIdent) {  // the fragment's 8 bf16 are contiguous: lo holds them in pairs
      const u32x4 v = *(const u32x4*)(smem + rbuf + 2 * (512 * (c0 + i) + 32 * r16 + 8 * kq));
      lo[0] = v.x; lo[1] = v.y; lo[2] = v.z; lo[3] = v.w;
      hi[0] = hi[1] = hi[2] = hi[3] = 0u;
      return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      asm volatile("" : "+v"(off[i][q]));
      lo[q] = lds_read_u16(rbuf + (off[i][q] & 0x7fffu));
      hi[q] = lds_read_u16(rbuf + ((off[i][q] >> 16) & 0x7fffu));
    }
  };
  uint32_t lo[4], hi[4];
  gather(0, lo, hi);
  float u[8];
  GridCell g[8];
#pragma unroll
  for (int i = 0; i <= NP; ++i) {
    float v[8];
    if (i < NP) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (lo[q] | (hi[q] << 16)) ^ (kIdent ? off[i][q] : off[i][q] & 0x80008000u);
      const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      if (i + 1 < NP) gather(i + 1, lo, hi);
      const floatx4 y0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb0, zero, 0, 0, 0);
      const floatx4 y1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb1, zero, 0, 0, 0);
      // y0[e], y1[e]: A row 4 kq + e at columns r16 and r16 + 16, i.e.
      // positions 512 c + 128 kq + 32 e + r16 (+ 16)
      v[0] = y0[0]; v[1] = y0[1]; v[2] = y0[2]; v[3] = y0[3];
      v[4] = y1[0]; v[5] = y1[1]; v[6] = y1[2]; v[7] = y1[3];
    }
    if (kQuant && i > 0) {  // the codes of pair i - 1
      const int base = 512 * (c0 + i - 1) + 128 * kq + r16;  // position of element 0
#pragma unroll
      for (int e = 0; e < 8; ++e)
        smem[cbuf + base + 32 * (e & 3) + 16 * (e >> 2)] = (char)(g[e].base + (g[e].t < u[e] ? 1 : 0));
    }
    if (i < NP) {
      group_stages<G>(v[0], v[1], v[2], v[3]);
      group_stages<G>(v[4], v[5], v[6], v[7]);
      if constexpr (G == 8) {  // groups t and t ^ 4 sit in lanes l and l ^ 16
#pragma clang fp contract(off)
        const float sg = (lane & 16) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = xor_partner<16>(v[e]) + v[e] * sg;
      }
      const int base = 512 * (c0 + i) + 128 * kq + r16;
      if constexpr (!kQuant) {  // fp16 x' into the staging buffer
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *(uint16_t*)(smem + cbuf + 2 * (base + 32 * (e & 3) + 16 * (e >> 2))) = f32_to_f16_rne(v[e] * a.inv_sqrt_h);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u[e] = v[e] * alpha;
          g[e] = *(const GridCell*)(smem + grid_addr(u[e], a.ga, a.gb, top, a.grid_bias));
        }
        if constexpr (kX) {
#pragma unroll
          for (int e = 0; e < 8; ++e) xr[base + 32 * (e & 3) + 16 * (e >> 2)] = v[e] * a.inv_sqrt_h;
        }
      }
    }
    // one pair at a time: hoisting later gathers would hold their registers
    // and cost occupancy
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The row's staged output: 16-code words for the codebook modes, 16-byte
// pieces of fp16 x' for kRotF16; threads t0, t0 + NT, ... of the row's team
// (a fixed trip count, so the loop unrolls and the code words keep their
// own aligned stores).
template <int MODE, int BITS, int D, int NT>
__device__ __forceinline__ void store_row(const RowArgs& a, const char* smem, uint32_t cbuf,
                                          long long row, int t0) {
  if constexpr (MODE == kRotF16) {
    static_assert((D / 8) % NT == 0, "whole rounds of 16-byte pieces");
    uint4* const out = (uint4*)(a.xrot_f16 + (size_t)row * D);
#pragma unroll
    for (int s = 0; s < D / 8 / NT; ++s) out[s * NT + t0] = *(const uint4*)(smem + cbuf + (s * NT + t0) * 16);
  } else {
    static_assert((D / kSlot) % NT == 0, "whole rounds of code words");
    uint8_t* const out = a.idx_out + (size_t)row * ((size_t)D * BITS / 8);
#pragma unroll
    for (int s = 0; s < D / kSlot / NT; ++s) {
      const int slot = s * NT + t0;
      const u32x4 cw = *(const u32x4*)(smem + cbuf + slot * 16);
      const uint32_t ww[4] = {cw.x, cw.y, cw.z, cw.w};
      int idx[kSlot];
#pragma unroll
      for (int i = 0; i < kSlot; ++i) idx[i] = (int)((ww[i >> 2] >> (8 * (i & 3))) & 0xffu);
      store_indices<BITS>(out, slot, idx);
    }
  }
}

// Rows of 512 C coordinates, one wave per row.  kX: also write the debug
// copy of x' (activation mode; a separate instantiation, so the plain kernel
// carries none of its registers).  The occupancy hints are the register
// budgets these instances meet without spills (hipcc's resource report):
// four waves per SIMD up to 3072 coordinates except with 2-bit codes.
constexpr int mfma_rows_waves(int bits, int c, bool x) {
  return x ? (c <= 4 ? 3 : 2) : (c <= 6 && bits != 2 ? 4 : 3);
}
template <int MODE, int BITS, int G, int C, bool kX, bool kIdent>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(mfma_rows_waves(BITS, C, kX)))) void mfma_rows_kernel(RowArgs a) {
  static_assert(MODE == kAct || MODE == kWeight || MODE == kRotF16, "codebook modes and fp16 x'");
  constexpr bool kQuant = MODE != kRotF16;
  static_assert(C >= 1 && C <= 8, "rows of 512 C coordinates, C <= 8");
  static_assert(G == 2 || G == 4 || G == 8, "h = 64, 128 or 256");
  extern __shared__ __align__(16) char smem[];
  constexpr int kD = 512 * C;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t wbuf = (uint32_t)(a.grid_bytes + wave * a.wave_bytes);  // the row
  const uint32_t cbuf = wbuf + 2u * kD;  // one code byte (fp16 x' for kRotF16) per position
  const int r16 = lane & 15, kq = lane >> 4;
  const long long stride = (long long)gridDim.x * waves;
  long long row = (long long)blockIdx.x * waves + wave;

  bf16x8 hb0, hb1;
  hadamard32_operands(r16, kq, hb0, hb1);
  // Load order.  Global loads retire in order, so waits for the signs, pi
  // and the grid issued behind the row's loads wait for the row as well.
  // With pi = identity only the sign words precede the row (measured: 4096
  // rows of 3072, 11.3 -> 10.5 us).  A random pi is 4 bytes per coordinate
  // that every wave reads whole; issued by all waves at once ahead of the
  // rows those reads contend in L2 (14.7 -> 18.9 us), so there the row goes
  // first.  The row load is unconditional (a spare wave reads the last row)
  // so that the compiler counts it on every path.
  uint32_t off[C][4];
  RowRegs<uint16_t, C> pre;
  if constexpr (kIdent) {
    pair_offsets<C, kIdent>(a, 0, r16, kq, off);
    if constexpr (kQuant) build_grid(a, smem);
    pre.load(a, row < a.rows ? row : a.rows - 1, lane);
  } else {
    pre.load(a, row < a.rows ? row : a.rows - 1, lane);
    pair_offsets<C, kIdent>(a, 0, r16, kq, off);
    if constexpr (kQuant) build_grid(a, smem);
  }
  __syncthreads();

  for (; row < a.rows; row += stride) {
    float ssx = 0.0f;
    if constexpr (kQuant) ssx = pre.sumsq(a, lane);
#pragma unroll
    for (int j = 0; j < C; ++j) *(u32x4*)(smem + wbuf + (lane + kWave * j) * 16) = pre.c[j];
    if (row + stride < a.rows) pre.load(a, row + stride, lane);
    float alpha = 0.0f;
    if constexpr (kQuant) alpha = row_alpha<MODE, true>(a, wave_sum(ssx), row, lane);
    wave_lds_sync();
    mfma_pairs<MODE, G, C, kX, kIdent>(a, wbuf, cbuf, 0, off, hb0, hb1, alpha,
                               kX ? a.xrot_f32 + row * kD : nullptr, lane);
    wave_lds_sync();  // the row's codes (or fp16 x') are in the staging buffer
    store_row<MODE, BITS, kD, kWave>(a, smem, cbuf, row, lane);
    wave_lds_sync();  // every lane has read its gathers and codes before the next row lands
  }
}

// Rows of 2048 CW coordinates (4096 < d <= 16384), one 4-wave workgroup per
// row: wave w takes pairs CW w .. CW w + CW - 1, the squared norm comes from
// a fixed-order workgroup reduction of the loaded row.
template <int MODE, int BITS, int G, int CW, bool kX, bool kIdent>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kX ? 2 : (CW <= 6 ? 4 : 3)))) void mfma_long_kernel(RowArgs a) {
  static_assert(MODE == kAct || MODE == kWeight, "codebook modes");
  static_assert(G == 2 || G == 4 || G == 8, "h = 64, 128 or 256");
  extern __shared__ __align__(16) char smem[];
  constexpr int kD = 2048 * CW;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  float* const red = (float*)(smem + a.grid_bytes);        // four wave sums
  const uint32_t rbuf = (uint32_t)a.grid_bytes + 16u;       // the row
  const uint32_t cbuf = rbuf + 2u * kD;                     // one code byte per position
  const int r16 = lane & 15, kq = lane >> 4;

  bf16x8 hb0, hb1;
  hadamard32_operands(r16, kq, hb0, hb1);
  // thread t loads 16-byte chunks t + 256 i of the row
  u32x4 pre[CW];
  auto load = [&](long long rr) {
    const u32x4* src = (const u32x4*)((const char*)a.in + (size_t)rr * kD * 2);
#pragma unroll
    for (int i = 0; i < CW; ++i) pre[i] = __builtin_nontemporal_load(src + t + 256 * i);
  };
  // the load order of the row kernel (the launch gives every workgroup a
  // row)
  long long row = blockIdx.x;
  uint32_t off[CW][4];
  if constexpr (kIdent) {
    pair_offsets<CW, kIdent>(a, CW * wave, r16, kq, off);
    build_grid(a, smem);
    load(row);
  } else {
    load(row);
    pair_offsets<CW, kIdent>(a, CW * wave, r16, kq, off);
    build_grid(a, smem);
  }

  for (; row < a.rows; row += gridDim.x) {
    float ssx = 0.0f;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      ssx = RowRegs<uint16_t, 1>::chunk_sumsq(pre[i], ssx);
      *(u32x4*)(smem + rbuf + (t + 256 * i) * 16) = pre[i];
    }
    if (row + gridDim.x < a.rows) load(row + gridDim.x);
    const float ws = wave_sum(ssx);
    if (lane == 0) red[wave] = ws;
    __syncthreads();  // the row, the wave sums (and, first time, the grid) are in LDS
    const float alpha = row_alpha<MODE, true>(a, (red[0] + red[1]) + (red[2] + red[3]), row, t);
    mfma_pairs<MODE, G, CW, kX, kIdent>(a, rbuf, cbuf, CW * wave, off, hb0, hb1, alpha,
                                kX ? a.xrot_f32 + row * kD : nullptr, lane);
    __syncthreads();  // every wave's codes are in the byte buffer
    store_row<MODE, BITS, kD, 256>(a, smem, cbuf, row, t);
    __syncthreads();  // the buffers are free for the next row
  }
}

// LDS bytes per wave: the bf16 row and its code bytes (fp16 x' for the
// rotation).
template <int MODE, int C>
constexpr int mfma_wave_bytes() { return (MODE == kRotF16 ? 4 : 3) * 512 * C; }

template <int MODE, int BITS, int G, int C, bool kX>
hipError_t launch_mfma_typed(RowArgs a, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  a.wave_bytes = mfma_wave_bytes<MODE, C>();
  int waves = 4;
  while (waves > 1 && a.grid_bytes + waves * a.wave_bytes > di.max_lds) waves >>= 1;
  const int lds = a.grid_bytes + waves * a.wave_bytes;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  auto kern = a.perm_identity ? mfma_rows_kernel<MODE, BITS, G, C, kX, true>
                              : mfma_rows_kernel<MODE, BITS, G, C, kX, false>;
  static LaunchCache cache, cache_ident;
  int per_cu = 1;
  e = prepare_launch(a.perm_identity ? cache_ident : cache, (const void*)kern, waves * kWave, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long need = (a.rows + waves - 1) / waves;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(need < cap ? need : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(waves * kWave), lds, stream, a);
  return hipGetLastError();
}

template <int MODE, int BITS, int G, int CW, bool kX>
hipError_t launch_mfma_long_typed(const RowArgs& a, hipStream_t stream) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int lds = a.grid_bytes + 16 + 3 * 2048 * CW;
  if (lds > di.max_lds) return hipErrorInvalidValue;
  auto kern = a.perm_identity ? mfma_long_kernel<MODE, BITS, G, CW, kX, true>
                              : mfma_long_kernel<MODE, BITS, G, CW, kX, false>;
  static LaunchCache cache, cache_ident;
  int per_cu = 1;
  e = prepare_launch(a.perm_identity ? cache_ident : cache, (const void*)kern, 256, lds, &per_cu);
  if (e != hipSuccess) return e;
  const long long cap = (long long)di.n_cu * per_cu;
  const int blocks = (int)(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <int MODE, int BITS, int G, bool kX>
hipError_t launch_mfma_d(const RowArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 1024: return launch_mfma_typed<MODE, BITS, G, 2, kX>(a, stream);
    case 2048: return launch_mfma_typed<MODE, BITS, G, 4, kX>(a, stream);
    case 3072: return launch_mfma_typed<MODE, BITS, G, 6, kX>(a, stream);
    case 4096: return launch_mfma_typed<MODE, BITS, G, 8, kX>(a, stream);
  }
  if constexpr (MODE != kRotF16) {  // one workgroup per row
    switch (a.d) {
      case 8192: return launch_mfma_long_typed<MODE, BITS, G, 4, kX>(a, stream);
      case 12288: return launch_mfma_long_typed<MODE, BITS, G, 6, kX>(a, stream);
      case 16384: return launch_mfma_long_typed<MODE, BITS, G, 8, kX>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <int MODE, int BITS, int G>
hipError_t launch_mfma_h(const RowArgs& a, hipStream_t stream) {
  if constexpr (MODE == kAct) {
    if (a.xrot_f32) return launch_mfma_d<MODE, BITS, G, true>(a, stream);
  }
  return launch_mfma_d<MODE, BITS, G, false>(a, stream);
}



}  // namespace rows
}  // namespace orbit

namespace orbit {
namespace rows {

#define ORBIT_ROWS_MFMA(MODE, G)                                                 \
  template <>                                                                  \
  hipError_t launch_mfma<MODE, G>(const RowArgs& a, int bits, hipStream_t s) { \
    switch (bits) {                                                            \
      case 2: return launch_mfma_h<MODE, 2, G>(a, s);                          \
      case 3: return launch_mfma_h<MODE, 3, G>(a, s);                          \
      case 4: return launch_mfma_h<MODE, 4, G>(a, s);                          \
      case 6: return launch_mfma_h<MODE, 6, G>(a, s);                          \
      case 8: return launch_mfma_h<MODE, 8, G>(a, s);                          \
    }                                                                          \
    return hipErrorInvalidValue;                                               \
  }

}  // namespace rows
}  // namespace orbit

namespace orbit {
namespace rows {

// The fp16 rotation (no code width).
#define ORBIT_ROWS_MFMA_ROT(G)                                                     \
  template <>                                                                    \
  hipError_t launch_mfma<kRotF16, G>(const RowArgs& a, int, hipStream_t s) {     \
    return launch_mfma_d<kRotF16, 4, G, false>(a, s);                            \
  }

}  // namespace rows
}  // namespace orbit
