// Transposed-gather rotation (fp32 / fp16 out) and int8 / int4 pack kernels: bf16 rows, h = 64 (see rpbh_impl.h).
#include "rpbh_impl.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_FAST_PLAIN(kRotF32, 2)
ORBIT_ROWS_FAST_PLAIN(kRotF16, 2)
ORBIT_ROWS_FAST_PLAIN(kInt8, 2)
ORBIT_ROWS_FAST_PLAIN(kInt4, 2)
}  // namespace rows
}  // namespace orbit
