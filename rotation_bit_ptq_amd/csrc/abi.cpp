// C ABI of liborbit: argument validation and dispatch to the HIP kernels.
// Every check runs on the host before any HIP call, so a bad argument
// returns an error code with nothing enqueued.
#include <cmath>
#include <cstdint>
#include <vector>

#include "orbit_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

orbit_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ORBIT_OK;
  g_last_hip_error = (int)e;
  return ORBIT_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

orbit_status check_rot(const orbit_rpbh* rot, int64_t d) {
  if (!rot || !rot->perm || !rot->sign_bits || !aligned16(rot->perm)) return ORBIT_E_ARG;
  if (rot->gather && !aligned16(rot->gather)) return ORBIT_E_ARG;
  if (rot->d != d || d < 16 || d > ORBIT_MAX_D) return ORBIT_E_SHAPE;
  if (!pow2(rot->h) || rot->h < 16 || rot->h > 4096 || d % rot->h) return ORBIT_E_SHAPE;
  if (rot->h > 1024 && d > 4096) return ORBIT_E_SHAPE;  // long blocks: rows kept in registers
  return ORBIT_OK;
}

// The identity hint counts only with the plan that orbit_rpbh_build_gather
// built (and whose flags it derived from perm).
bool identity_hint(const orbit_rpbh* rot) {
  return rot->gather != nullptr && (rot->flags & ORBIT_RPBH_IDENTITY) != 0;
}

bool code_bits(int b) { return b == 1 || b == 2 || b == 3 || b == 4 || b == 6 || b == 8; }

// Ascending, finite, thresholds strictly between neighbouring centroids.
orbit_status check_codebook(const orbit_codebook* cb) {
  if (!cb || !code_bits(cb->bits)) return ORBIT_E_ARG;
  const int levels = 1 << cb->bits;
  for (int j = 0; j < levels; ++j)
    if (!std::isfinite(cb->centroids[j])) return ORBIT_E_ARG;
  for (int j = 0; j + 1 < levels; ++j) {
    const float t = cb->thresholds[j];
    if (!std::isfinite(t) || !(cb->centroids[j] < t) || !(t < cb->centroids[j + 1])) return ORBIT_E_ARG;
  }
  return ORBIT_OK;
}

// The kernels' cell of u: fma(u, a, b + 2^23) is a float in [2^23, 2^24)
// once clamped, i.e. rounded to an integer; a monotone map of u.
const float kMagic = 8388608.0f;
int cell_of(float u, float a, float b_magic, int cells) {
  float f = std::fmaf(u, a, b_magic);
  f = std::fmin(std::fmax(f, kMagic), kMagic + (float)(cells - 1));
  return (int)(f - kMagic);
}

// Smallest uniform grid over [-T, T] whose cells each hold at most one
// threshold, using exactly the float32 classification the kernel uses.
bool choose_grid(const orbit_codebook* cb, orbit::GridSearch* g) {
  const int n = (1 << cb->bits) - 1;
  float tmax = 0.0f;
  for (int j = 0; j < n; ++j) tmax = std::fmax(tmax, std::fabs(cb->thresholds[j]));
  const float T = tmax * 1.001f + 1e-6f;
  for (int cells = 8; cells <= orbit::kMaxGridCells; cells *= 2) {
    const float a = (float)cells / (2.0f * T), b = (float)cells / 2.0f + kMagic;
    bool ok = true;
    for (int j = 1; j < n && ok; ++j)
      ok = cell_of(cb->thresholds[j - 1], a, b, cells) < cell_of(cb->thresholds[j], a, b, cells);
    if (ok) {
      g->a = a;
      g->b = b;
      g->cells = cells;
      g->nthr = n;
      return true;
    }
  }
  return false;
}

orbit_status check_rows_in(const void* in, orbit_dtype dt, int64_t rows) {
  if (rows < 0) return ORBIT_E_SHAPE;
  if (dt != ORBIT_F32 && dt != ORBIT_BF16) return ORBIT_E_DTYPE;
  if (rows > 0 && (!in || !aligned16(in))) return ORBIT_E_ARG;
  return ORBIT_OK;
}

// Rotate + per-group pack of weight rows (int8 or int4 codes).
orbit_status group_pack(orbit::RowMode mode, const orbit_rpbh* rot, const void* W,
                        orbit_dtype w_dtype, int64_t N, int64_t K, int32_t group, int8_t* q_out,
                        uint16_t* scale_f16_out, hipStream_t stream) {
  orbit_status st = check_rot(rot, K);
  if (st != ORBIT_OK) return st;
  if ((st = check_rows_in(W, w_dtype, N)) != ORBIT_OK) return st;
  if (!pow2(group) || group < 16 || group > 1024 || K % group) return ORBIT_E_SHAPE;
  if (N > 0 && (!q_out || !scale_f16_out || !aligned16(q_out))) return ORBIT_E_ARG;
  orbit::RowJob job = {};
  job.mode = mode;
  job.in_dtype = w_dtype;
  job.rows = N;
  job.d = (int)K;
  job.h = rot->h;
  job.perm = rot->perm;
  job.gather = rot->gather;
  job.perm_identity = identity_hint(rot);
  job.sign_bits = rot->sign_bits;
  job.in = W;
  job.group = group;
  job.q_out = q_out;
  job.scale_out = scale_f16_out;
  return hip_status(orbit::launch_rows(job, stream));
}

// fp16 rotated activations x int8 (kind 1) or int4 (kind 2) weights.
orbit_status group_linear(int kind, const void* Xrot, orbit_dtype xrot_dtype, int64_t M, int64_t K,
                          const uint8_t* q, const uint16_t* scale_f16, int32_t group, int64_t N,
                          const void* bias, orbit_dtype bias_dtype, void* out,
                          orbit_dtype out_dtype, hipStream_t stream) {
  if (xrot_dtype != ORBIT_F16) return ORBIT_E_DTYPE;
  if (out_dtype != ORBIT_F32 && out_dtype != ORBIT_BF16) return ORBIT_E_DTYPE;
  if (bias && bias_dtype != ORBIT_F32 && bias_dtype != ORBIT_BF16) return ORBIT_E_DTYPE;
  if (group != 128) return ORBIT_E_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 128 || K > 65536 || K % 128) return ORBIT_E_SHAPE;
  if (M > 0 && N > 0) {
    if (!Xrot || !q || !scale_f16 || !out) return ORBIT_E_ARG;
    if (!aligned16(Xrot) || !aligned16(q) || !aligned16(out)) return ORBIT_E_ARG;
  }
  const int64_t ldb = kind == 2 ? K / 2 : K;
  if (M * K * 2 >= (1LL << 31) || N * ldb >= (1LL << 31)) return ORBIT_E_UNSUPPORTED;
  orbit::GemmJob job = {};
  job.kind = kind;
  job.M = M;
  job.N = N;
  job.K = K;
  job.a = (const uint8_t*)Xrot;
  job.b = q;
  job.scale_f16 = scale_f16;
  job.group = group;
  job.bias = bias;
  job.bias_dtype = bias_dtype;
  job.out = out;
  job.out_dtype = out_dtype;
  return hip_status(orbit::launch_gemm(job, stream));
}

}  // namespace

namespace orbit {

hipError_t device_info(DeviceInfo* out) {
  static std::atomic<int> lds_cache[64];
  static std::atomic<int> cu_cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cu_cache[dev].load(std::memory_order_acquire) > 0) {
    out->max_lds = lds_cache[dev].load(std::memory_order_relaxed);
    out->n_cu = cu_cache[dev].load(std::memory_order_relaxed);
    return hipSuccess;
  }
  e = hipDeviceGetAttribute(&out->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&out->n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    lds_cache[dev].store(out->max_lds, std::memory_order_relaxed);
    cu_cache[dev].store(out->n_cu, std::memory_order_release);
  }
  return hipSuccess;
}

hipError_t prepare_launch(LaunchCache& c, const void* kern, int threads, int lds, int* blocks_per_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (lds > 64 * 1024 && !(c.lds_raised.load(std::memory_order_acquire) & bit)) {
    DeviceInfo di;
    if ((e = device_info(&di)) != hipSuccess) return e;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, di.max_lds);
    if (e != hipSuccess) return e;
    c.lds_raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (blocks_per_cu) {
    const long long key = ((long long)dev << 32) | (unsigned)lds;
    if (c.occ_key.load(std::memory_order_acquire) == key) {
      *blocks_per_cu = c.occ_blocks.load(std::memory_order_relaxed);
    } else {
      int per_cu = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds);
      if (e != hipSuccess || per_cu < 1) per_cu = 1;
      c.occ_blocks.store(per_cu, std::memory_order_relaxed);
      c.occ_key.store(key, std::memory_order_release);
      *blocks_per_cu = per_cu;
    }
  }
  return hipSuccess;
}

}  // namespace orbit

extern "C" {

const char* orbit_status_string(orbit_status status) {
  switch (status) {
    case ORBIT_OK: return "ok";
    case ORBIT_E_ARG: return "invalid argument";
    case ORBIT_E_SHAPE: return "invalid shape";
    case ORBIT_E_DTYPE: return "unsupported dtype";
    case ORBIT_E_UNSUPPORTED: return "unsupported configuration";
    case ORBIT_E_HIP: return "HIP error";
  }
  return "unknown status";
}

orbit_status orbit_last_hip_error(int* hip_error_out) {
  if (!hip_error_out) return ORBIT_E_ARG;
  *hip_error_out = g_last_hip_error;
  return ORBIT_OK;
}

int64_t orbit_rpbh_gather_len(int32_t d, int32_t h) {
  if (d < 16 || d > ORBIT_MAX_D || !pow2(h) || h < 16 || h > 4096 || d % h) return 0;
  if (h > 1024 && d > 4096) return 0;
  return (int64_t)orbit::gather_len(d) + orbit::mfma_words_len(d, h) + orbit::scatter_len(d, h);
}

orbit_status orbit_rpbh_build_gather(orbit_rpbh* rot, uint16_t* out, hipStream_t stream) {
  if (!rot) return ORBIT_E_ARG;
  orbit_rpbh plain = *rot;
  plain.gather = nullptr;
  orbit_status st = check_rot(&plain, rot->d);
  if (st != ORBIT_OK) return st;
  if (!out || !aligned16(out)) return ORBIT_E_ARG;
  // the identity hint is derived here from perm itself, never trusted
  std::vector<int32_t> host((size_t)rot->d);
  hipError_t e = hipMemcpyAsync(host.data(), rot->perm, host.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e);
  // the plan's sections assume a permutation (the scatter section has one
  // entry per input coordinate)
  std::vector<char> seen((size_t)rot->d, 0);
  bool ident = true;
  for (int32_t k = 0; k < rot->d; ++k) {
    const int32_t p = host[(size_t)k];
    if (p < 0 || p >= rot->d || seen[(size_t)p]) return ORBIT_E_ARG;
    seen[(size_t)p] = 1;
    ident = ident && p == k;
  }
  rot->flags = ident ? ORBIT_RPBH_IDENTITY : 0;
  return hip_status(orbit::launch_gather_plan(rot->d, rot->h, rot->perm, rot->sign_bits, out, stream));
}

orbit_status orbit_pack_weights(const orbit_rpbh* rot, const orbit_codebook* cw, const void* W,
                                orbit_dtype w_dtype, int64_t d_out, int64_t d_in, uint8_t* idx_out,
                                uint16_t* r_bf16_out, hipStream_t stream) {
  orbit_status st = check_rot(rot, d_in);
  if (st != ORBIT_OK) return st;
  if ((st = check_codebook(cw)) != ORBIT_OK) return st;
  if ((st = check_rows_in(W, w_dtype, d_out)) != ORBIT_OK) return st;
  if (d_out > 0 && (!idx_out || !r_bf16_out || !aligned16(idx_out))) return ORBIT_E_ARG;
  orbit::RowJob job = {};
  if (!choose_grid(cw, &job.grid)) return ORBIT_E_UNSUPPORTED;
  job.mode = orbit::RowMode::kWeightQuant;
  job.in_dtype = w_dtype;
  job.rows = d_out;
  job.d = (int)d_in;
  job.h = rot->h;
  job.perm = rot->perm;
  job.gather = rot->gather;
  job.perm_identity = identity_hint(rot);
  job.sign_bits = rot->sign_bits;
  job.in = W;
  job.bits = cw->bits;
  job.thresholds = cw->thresholds;
  job.idx_out = idx_out;
  job.norm_bf16_out = r_bf16_out;
  return hip_status(orbit::launch_rows(job, stream));
}

orbit_status orbit_quant_act(const orbit_rpbh* rot, const orbit_codebook* ca, const void* X,
                             orbit_dtype x_dtype, int64_t M, int64_t d, float eps, uint8_t* idx_out,
                             float* s_out, float* xrot_f32_debug, hipStream_t stream) {
  orbit_status st = check_rot(rot, d);
  if (st != ORBIT_OK) return st;
  if ((st = check_codebook(ca)) != ORBIT_OK) return st;
  if ((st = check_rows_in(X, x_dtype, M)) != ORBIT_OK) return st;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ORBIT_E_ARG;
  if (M > 0 && (!idx_out || !s_out || !aligned16(idx_out))) return ORBIT_E_ARG;
  if (xrot_f32_debug && !aligned16(xrot_f32_debug)) return ORBIT_E_ARG;
  orbit::RowJob job = {};
  if (!choose_grid(ca, &job.grid)) return ORBIT_E_UNSUPPORTED;
  job.mode = orbit::RowMode::kActQuant;
  job.in_dtype = x_dtype;
  job.rows = M;
  job.d = (int)d;
  job.h = rot->h;
  job.perm = rot->perm;
  job.gather = rot->gather;
  job.perm_identity = identity_hint(rot);
  job.sign_bits = rot->sign_bits;
  job.in = X;
  job.bits = ca->bits;
  job.thresholds = ca->thresholds;
  job.eps = eps;
  job.idx_out = idx_out;
  job.norm_f32_out = s_out;
  job.xrot_f32_out = xrot_f32_debug;
  return hip_status(orbit::launch_rows(job, stream));
}

orbit_status orbit_rotate(const orbit_rpbh* rot, const void* X, orbit_dtype x_dtype, int64_t M,
                          int64_t d, void* out, orbit_dtype out_dtype, hipStream_t stream) {
  orbit_status st = check_rot(rot, d);
  if (st != ORBIT_OK) return st;
  if ((st = check_rows_in(X, x_dtype, M)) != ORBIT_OK) return st;
  if (out_dtype != ORBIT_F32 && out_dtype != ORBIT_F16) return ORBIT_E_DTYPE;
  if (M > 0 && (!out || !aligned16(out))) return ORBIT_E_ARG;
  orbit::RowJob job = {};
  job.mode = orbit::RowMode::kRotate;
  job.in_dtype = x_dtype;
  job.out_dtype = out_dtype;
  job.rows = M;
  job.d = (int)d;
  job.h = rot->h;
  job.perm = rot->perm;
  job.gather = rot->gather;
  job.perm_identity = identity_hint(rot);
  job.sign_bits = rot->sign_bits;
  job.in = X;
  if (out_dtype == ORBIT_F32) job.xrot_f32_out = (float*)out; else job.rot_out = out;
  return hip_status(orbit::launch_rows(job, stream));
}

orbit_status orbit_int8_pack_weights(const orbit_rpbh* rot, const void* W, orbit_dtype w_dtype,
                                     int64_t N, int64_t K, int32_t group, int8_t* q_out,
                                     uint16_t* scale_f16_out, hipStream_t stream) {
  return group_pack(orbit::RowMode::kInt8Pack, rot, W, w_dtype, N, K, group, q_out,
                    scale_f16_out, stream);
}

orbit_status orbit_int4_pack_weights(const orbit_rpbh* rot, const void* W, orbit_dtype w_dtype,
                                     int64_t N, int64_t K, int32_t group, uint8_t* q_out,
                                     uint16_t* scale_f16_out, hipStream_t stream) {
  return group_pack(orbit::RowMode::kInt4Pack, rot, W, w_dtype, N, K, group, (int8_t*)q_out,
                    scale_f16_out, stream);
}

orbit_status orbit_int4_linear(const void* Xrot, orbit_dtype xrot_dtype, int64_t M, int64_t K,
                               const uint8_t* q, const uint16_t* scale_f16, int32_t group,
                               int64_t N, const void* bias, orbit_dtype bias_dtype, void* out,
                               orbit_dtype out_dtype, hipStream_t stream) {
  return group_linear(2, Xrot, xrot_dtype, M, K, q, scale_f16, group, N, bias, bias_dtype, out,
                      out_dtype, stream);
}

orbit_status orbit_int8_linear(const void* Xrot, orbit_dtype xrot_dtype, int64_t M, int64_t K,
                               const int8_t* q, const uint16_t* scale_f16, int32_t group, int64_t N,
                               const void* bias, orbit_dtype bias_dtype, void* out,
                               orbit_dtype out_dtype, hipStream_t stream) {
  return group_linear(1, Xrot, xrot_dtype, M, K, (const uint8_t*)q, scale_f16, group, N, bias,
                      bias_dtype, out, out_dtype, stream);
}

orbit_status orbit_qlinear_act(const uint8_t* idx_a, const float* s, const orbit_codebook* ca,
                               const uint8_t* idx_w, const uint16_t* r_bf16,
                               const orbit_codebook* cw, const void* bias, orbit_dtype bias_dtype,
                               int64_t M, int64_t N, int64_t K, void* out, orbit_dtype out_dtype,
                               orbit_act act, hipStream_t stream) {
  orbit_status st;
  if (act != ORBIT_ACT_NONE && act != ORBIT_ACT_GELU) return ORBIT_E_ARG;
  if ((st = check_codebook(ca)) != ORBIT_OK) return st;
  if ((st = check_codebook(cw)) != ORBIT_OK) return st;
  if (ca->bits == 1 || cw->bits == 1) return ORBIT_E_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 128 || K > 65536 || K % 128) return ORBIT_E_SHAPE;
  if (out_dtype != ORBIT_F32 && out_dtype != ORBIT_BF16) return ORBIT_E_DTYPE;
  if (bias && bias_dtype != ORBIT_F32 && bias_dtype != ORBIT_BF16) return ORBIT_E_DTYPE;
  if (M > 0 && N > 0) {
    if (!idx_a || !s || !idx_w || !r_bf16 || !out) return ORBIT_E_ARG;
    if (!aligned16(idx_a) || !aligned16(idx_w) || !aligned16(out)) return ORBIT_E_ARG;
  }
  // operand row offsets are 32-bit inside the kernels
  if (M * (K * ca->bits / 8) >= (1LL << 31) || N * (K * cw->bits / 8) >= (1LL << 31))
    return ORBIT_E_UNSUPPORTED;
  orbit::GemmJob job = {};
  job.kind = 0;
  job.M = M;
  job.N = N;
  job.K = K;
  job.a = idx_a;
  job.b = idx_w;
  job.bits_a = ca->bits;
  job.bits_b = cw->bits;
  job.cent_a = ca->centroids;
  job.cent_b = cw->centroids;
  job.s = s;
  job.r_bf16 = r_bf16;
  job.bias = bias;
  job.bias_dtype = bias_dtype;
  job.out = out;
  job.out_dtype = out_dtype;
  job.act = act;
  return hip_status(orbit::launch_gemm(job, stream));
}

orbit_status orbit_qlinear(const uint8_t* idx_a, const float* s, const orbit_codebook* ca,
                           const uint8_t* idx_w, const uint16_t* r_bf16, const orbit_codebook* cw,
                           const void* bias, orbit_dtype bias_dtype, int64_t M, int64_t N, int64_t K,
                           void* out, orbit_dtype out_dtype, hipStream_t stream) {
  return orbit_qlinear_act(idx_a, s, ca, idx_w, r_bf16, cw, bias, bias_dtype, M, N, K, out,
                           out_dtype, ORBIT_ACT_NONE, stream);
}

}  // extern "C"
