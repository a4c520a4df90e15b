// Transposed-gather rotation (fp32 / fp16 out) and int8 / int4 pack kernels: bf16 rows, h = 128 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST_PLAIN(kRotF32, 3)
ORBIT_ROWS_FAST_PLAIN(kRotF16, 3)
ORBIT_ROWS_FAST_PLAIN(kInt8, 3)
ORBIT_ROWS_FAST_PLAIN(kInt4, 3)
}  // namespace rows
}  // namespace orbit
