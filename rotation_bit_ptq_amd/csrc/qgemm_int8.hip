// Int8 and int4 weight-only GEMM kernels on rotated fp16 activations (see
// qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
namespace {

// Large products take the LDS-staged kernel (256 x 256 tiles, a ring of
// three 64-k chunks); products with fewer tiles than that fills keep the
// register-fed kernel and its smaller tiles.  The staged kernel reads each
// fp16 group scale through the aligned dword that holds it, so it also needs
// a 4-byte aligned scale array with an even number of entries (else the last
// dword would reach past the array).
template <class OpB>
hipError_t launch_weight_only(GemmArgs& g, hipStream_t stream) {
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
