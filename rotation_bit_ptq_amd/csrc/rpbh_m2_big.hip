// Matrix-core rotate + quantize for Hadamard blocks of 512 .. 4096 coordinates
// (the full RHT) on bf16 rows of 2048 or 4096: activation, weight and fp16
// rotation modes (see rpbh_mfma2.h, big_kernel).
#include "rpbh_mfma2.h"

namespace orbit {
namespace rows {
ORBIT_ROWS_M2_BIG(kAct)
ORBIT_ROWS_M2_BIG(kWeight)
ORBIT_ROWS_M2_BIG_ROT
}  // namespace rows
}  // namespace orbit
