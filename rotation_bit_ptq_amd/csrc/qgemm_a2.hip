// Decode-GEMM kernels for 2-bit activation codes (see qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
ORBIT_DEFINE_LAUNCH_CODES_B(2)
}  // namespace qgemm
}  // namespace orbit
