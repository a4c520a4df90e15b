// Packed-run matrix-core fp16 rotation kernels: bf16 rows, h = 128 and 256 (see rpbh_mfma2.h).
#include "rpbh_mfma2.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_M2_ROT(4)
ORBIT_ROWS_M2_ROT(8)
}  // namespace rows
}  // namespace orbit
