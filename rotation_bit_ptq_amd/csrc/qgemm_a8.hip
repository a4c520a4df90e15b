// Decode-GEMM kernels for 8-bit activation codes (see qgemm_impl.h).
#include "qgemm_impl.h"

namespace orbit {
namespace qgemm {
ORBIT_DEFINE_LAUNCH_CODES_B(8)
}  // namespace qgemm
}  // namespace orbit
