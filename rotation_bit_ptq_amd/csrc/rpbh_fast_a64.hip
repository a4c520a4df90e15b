// Transposed-gather rotate + quantize kernels: bf16 activation rows, h = 64 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST(kAct, 2)
}  // namespace rows
}  // namespace orbit
