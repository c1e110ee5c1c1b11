// Matrix-vector kernel instances for Q8_0 rows.
#include "matvec_kern.h"

namespace moe {
MOE_MV_INSTANCES(MOE_FMT_Q8_0)
MOE_MV_DOWN_TOK_INSTANCES(MOE_FMT_Q8_0)
}  // namespace moe
