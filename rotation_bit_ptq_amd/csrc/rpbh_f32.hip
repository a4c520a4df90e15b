// Row kernels for fp32 rows (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_QUANT_MODE(float, kAct)
ORBIT_ROWS_QUANT_MODE(float, kWeight)
ORBIT_ROWS_PLAIN_MODE(float, kRotF32)
ORBIT_ROWS_PLAIN_MODE(float, kRotF16)
ORBIT_ROWS_PLAIN_MODE(float, kInt8)
ORBIT_ROWS_PLAIN_MODE(float, kInt4)
}  // namespace rows
}  // namespace orbit
