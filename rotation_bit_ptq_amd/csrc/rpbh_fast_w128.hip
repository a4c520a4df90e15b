// Transposed-gather rotate + quantize kernels: bf16 weight rows, h = 128 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST(kWeight, 3)
}  // namespace rows
}  // namespace orbit
