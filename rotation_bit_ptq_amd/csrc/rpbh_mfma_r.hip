// Matrix-core rotation kernels: bf16 rows to fp16 x', h = 64, 128, 256 (see rpbh_mfma.h).
#include "rpbh_mfma.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_MFMA_ROT(2)
ORBIT_ROWS_MFMA_ROT(4)
ORBIT_ROWS_MFMA_ROT(8)
}  // namespace rows
}  // namespace orbit
