// Transposed-gather rotate + quantize kernels: bf16 weight rows, h = 64 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST(kWeight, 2)
}  // namespace rows
}  // namespace orbit
