// Transposed-gather rotate + quantize kernels: bf16 activation rows, h = 128 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST(kAct, 3)
}  // namespace rows
}  // namespace orbit
