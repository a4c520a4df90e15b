// Rotate + quantize kernels for bf16 activation rows (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_QUANT_MODE(uint16_t, kAct)
}  // namespace rows
}  // namespace orbit
