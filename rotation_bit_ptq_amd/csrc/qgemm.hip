// Host entry of the decode GEMMs: fills the kernel arguments and picks the
// instantiation for the operand widths (kernels in qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace {

uint16_t host_f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace

hipError_t launch_gemm(const GemmJob& job, hipStream_t stream) {
  using namespace qgemm;
  GemmArgs g = {};
  g.M = job.M;
  g.N = job.N;
  g.K = job.K;
  g.a = job.a;
  g.b = job.b;
  g.s = job.s;
  g.r_bf16 = job.r_bf16;
  g.scale_f16 = job.scale_f16;
  g.inv_k = (float)(1.0 / (double)job.K);
  g.bias = job.bias;
  g.bias_dtype = job.bias_dtype;
  g.out = job.out;
  g.out_dtype = job.out_dtype;
  g.act = job.act;
  if (job.M == 0 || job.N == 0) return hipSuccess;
  if (job.kind == 0) {
    g.lda = job.K * job.bits_a / 8;
    g.ldb = job.K * job.bits_b / 8;
    bool same = job.bits_a == job.bits_b;
    for (int i = 0; i < (1 << job.bits_a); ++i) g.cent_a[i] = host_f32_to_f16_rne(job.cent_a[i]);
    for (int i = 0; i < (1 << job.bits_b); ++i) {
      g.cent_b[i] = host_f32_to_f16_rne(job.cent_b[i]);
      if (same && g.cent_b[i] != g.cent_a[i]) same = false;
    }
    switch (job.bits_a) {
      case 2: return launch_codes_b<2>(g, job.bits_b, stream, same);
      case 3: return launch_codes_b<3>(g, job.bits_b, stream, same);
      case 4: return launch_codes_b<4>(g, job.bits_b, stream, same);
      case 6: return launch_codes_b<6>(g, job.bits_b, stream, same);
      case 8: return launch_codes_b<8>(g, job.bits_b, stream, same);
    }
    return hipErrorInvalidValue;
  }
  g.lda = job.K * 2;
  g.ldb = job.kind == 2 ? job.K / 2 : job.K;
  g.groups_per_row = (int)(job.K / job.group);
  g.table_a_offset = 0;
  g.table_b_offset = 0;
  return job.kind == 2 ? launch_int4(g, stream) : launch_int8(g, stream);
}

}  // namespace orbit
