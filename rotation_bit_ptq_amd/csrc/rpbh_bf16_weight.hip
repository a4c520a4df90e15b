// Rotate + quantize kernels for bf16 weight rows (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_QUANT_MODE(uint16_t, kWeight)
}  // namespace rows
}  // namespace orbit
