// Matrix-core rotate + quantize kernels: bf16 activation rows, h = 128 (see rpbh_mfma.h).
#include "rpbh_mfma.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_MFMA(kAct, 4)
}  // namespace rows
}  // namespace orbit
