// Matrix-vector kernel instances for NVFP4 rows (E2M1 codes, two E4M3 scales
// per block of 32, an fp32 scale per tensor).
#include "matvec_kern.h"

namespace moe {
MOE_MV_INSTANCES(MOE_FMT_NVFP4)
MOE_MV_DOWN_TOK_INSTANCES(MOE_FMT_NVFP4)
}  // namespace moe
