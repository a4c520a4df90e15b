// Int8 and int4 weight-only GEMM kernels on rotated fp16 activations (see
// qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
hipError_t launch_int8(GemmArgs& g, hipStream_t stream) {
  return launch_shape<1, F16Op, I8Op>(g, 0, stream);
}
hipError_t launch_int4(GemmArgs& g, hipStream_t stream) {
  return launch_shape<1, F16Op, I4Op>(g, 0, stream);
}
}  // namespace qgemm
}  // namespace orbit
