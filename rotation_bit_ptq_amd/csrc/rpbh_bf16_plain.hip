// Rotation-only and int8 / int4 pack kernels for bf16 rows (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_PLAIN_MODE(uint16_t, kRotF32)
ORBIT_ROWS_PLAIN_MODE(uint16_t, kRotF16)
ORBIT_ROWS_PLAIN_MODE(uint16_t, kInt8)
ORBIT_ROWS_PLAIN_MODE(uint16_t, kInt4)
}  // namespace rows
}  // namespace orbit
