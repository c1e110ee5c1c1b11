// Matrix-vector kernel instances for Q5_1 rows.
#include "matvec_kern.h"

namespace moe {
MOE_MV_INSTANCES(MOE_FMT_Q5_1)
MOE_MV_DOWN_TOK_INSTANCES(MOE_FMT_Q5_1)
}  // namespace moe
