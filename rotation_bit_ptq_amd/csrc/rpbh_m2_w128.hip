// Packed-code matrix-core rotate + quantize kernels: bf16 rows, weight mode, h = 128 (see rpbh_mfma2.h).
#include "rpbh_mfma2.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_M2(kWeight, 4)
}  // namespace rows
}  // namespace orbit
