// Transposed-gather rotation (fp32 / fp16 out) and int8 / int4 pack kernels: bf16 rows, h = 256 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST_PLAIN(kRotF32, 4)
ORBIT_ROWS_FAST_PLAIN(kRotF16, 4)
ORBIT_ROWS_FAST_PLAIN(kInt8, 4)
ORBIT_ROWS_FAST_PLAIN(kInt4, 4)
}  // namespace rows
}  // namespace orbit
