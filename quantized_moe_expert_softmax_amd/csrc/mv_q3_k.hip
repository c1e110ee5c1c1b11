// Matrix-vector kernel instances for Q3_K rows.
#include "matvec_kern.h"

namespace moe {
MOE_MV_INSTANCES(MOE_FMT_Q3_K)
MOE_MV_DOWN_TOK_KQ_INSTANCES(MOE_FMT_Q3_K)
}  // namespace moe
