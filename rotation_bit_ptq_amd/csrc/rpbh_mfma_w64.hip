// Matrix-core rotate + quantize kernels: bf16 weight rows, h = 64 (see rpbh_mfma.h).
#include "rpbh_mfma.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_MFMA(kWeight, 2)
}  // namespace rows
}  // namespace orbit
