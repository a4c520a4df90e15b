// Transposed-gather rotate + quantize kernels: bf16 weight rows, h = 256 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST(kWeight, 4)
}  // namespace rows
}  // namespace orbit
